// Internal launchers shared by the C-ABI layer (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// router.hip
int router_split(int64_t T, int d, int E, int dtype);
size_t route_ws_bytes(int64_t T, int d, int E);
// n_group > 1: group-limited routing (topk_group groups of E / n_group).
hipError_t launch_route(const void* X, int dtype, int64_t T, int d, const void* Wg, int E,
                        const float* bias, const float* offset, int score, int k, int renorm,
                        int n_group, int topk_group, float* logits, int32_t* ids, float* w,
                        float* prob_sum, void* ws, hipStream_t s, float* ent_part = nullptr,
                        int n_backup = 0, int32_t* backup = nullptr);
hipError_t launch_bias_update(const int32_t* counts, int64_t T, int k, int E, float gamma,
                              float* bias, hipStream_t s);
// {token entropy, load entropy, load CV, drop rate}; ent_part holds one
// partial per block of four tokens (written by launch_route).
hipError_t launch_router_health(const int32_t* counts, const int32_t* n_kept,
                                const float* ent_part, int64_t T, int k, int E, double* out,
                                hipStream_t s);
// Expert-choice routing: every expert takes C (<= T) tokens.  Writes
// offsets[E+1] (+ offsets[E+1] = E*C + tail_rows when tail_rows > 0),
// slot_row and gates [T][E] (slot t*E + e; -1 / 0 where not taken) and,
// when non-NULL, counts[E] (= C), n_kept (= E*C), sorted_slot[E*C],
// row_token[E*C + tail_rows] (the tail rows map to tokens 0..tail_rows-1).
size_t route_ec_ws_bytes(int64_t T, int d, int E);
hipError_t launch_route_ec(const void* X, int dtype, int64_t T, int d, const void* Wg, int E,
                           const float* offset, int score, int C, float* logits,
                           int32_t* offsets, int32_t* counts, int32_t* n_kept,
                           int32_t* sorted_slot, int32_t* slot_row, float* gates,
                           int32_t* row_token, int tail_rows, void* ws, hipStream_t s);
hipError_t launch_balance(const int32_t* counts, const float* prob_sum, int64_t T, int k, int E,
                          double* out, hipStream_t s);

// align.hip
size_t dispatch_ws_bytes(int64_t T, int k, int E);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_dispatch(const int32_t* ids, int64_t T, int k, int E, int64_t cap, int tail_rows,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                           int32_t* slot_row, int32_t* n_kept, int32_t* row_token, void* ws,
                           hipStream_t s);
// One backup round after the capacity drop (cap > 0): launch_dispatch's
// slot_row / sorted_slot / offsets / n_kept / row_token are rewritten with
// the dropped slots' accepted backup experts (backup[T][nb], -1 = none).
// ws: at least reroute_ws_bytes(T, k, E).
size_t reroute_ws_bytes(int64_t T, int k, int E);
hipError_t launch_reroute(const int32_t* ids, const int32_t* backup, int nb, int64_t T, int k,
                          int E, int64_t cap, int tail_rows, const int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                          int32_t* n_kept, int32_t* row_token, void* ws, hipStream_t s);
hipError_t launch_gather(const void* X, const int32_t* sorted_slot, const int32_t* n_kept,
                         int64_t Tk, int k, int d, int elem_bytes, void* Xs, hipStream_t s);

// gemm.hip
size_t ffn_ws_bytes(int64_t max_rows, int G, int d, int F, int dtype);
// Router logits on the tiled GEMM kernel (bf16, E a multiple of 64):
// part[z][T][E] for the `split` K-splits z.
bool router_gemm_ok(int dtype, int64_t T, int d, int E, int split);
int router_gemm_tiles(int64_t T, int E);
size_t router_gemm_ws_bytes(int64_t T, int d, int E, int split);
hipError_t launch_router_gemm(const void* X, const void* Wg, int64_t T, int d, int E, int split,
                              float* part, void* ws, hipStream_t s);
// Per-output-channel scales of FP8 (E4M3) weights: s1, s3 [G][F], s2 [G][d]
// for the routed groups, s1l, s3l [F], s2l [d] for group g_last.
struct WeightScales {
  const float *s1, *s3, *s2, *s1l, *s3l, *s2l;
};
// Yrows receives the complete down projection.
// q != NULL: W1/W3/W2 (and the g_last matrices) hold E4M3 codes, A is bf16.
// a_rows: rows A holds (row_token indexes them), or -1 if not known; with a
// bound the large bf16 tiles may address A through 32-bit offsets.
hipError_t launch_grouped_ffn(const void* A, const int32_t* row_token, const int32_t* offsets,
                              int G, const void* W1, const void* W3, const void* W2,
                              const void* W1l, const void* W3l, const void* W2l, int g_last,
                              int dtype, int d, int F, int64_t max_rows, float* Yrows, void* ws,
                              hipStream_t s, const WeightScales* q = nullptr,
                              int64_t a_rows = -1);

// combine.hip
hipError_t launch_combine(const float* Yrows, const int32_t* slot_row, const float* w, int64_t T,
                          int k, int d, const float* shared, const int32_t* shared_row0, void* Y,
                          int dtype, hipStream_t s);

// timing.hip: records a phase-boundary event when timing is enabled.
void timing_mark(const char* name, hipStream_t s, int first = 0);

}  // namespace moe
