// C-ABI entry points: host-side validation, workspace carving, launches.
// Nothing here allocates, frees or synchronises device memory.
#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

#define MOE_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_dtype(int dtype) {
  MOE_REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_EINVAL, "dtype %d is not MOE_F32 or MOE_BF16", dtype);
  return MOE_OK;
}

int check_router_dims(int64_t T, int d, int E, int k) {
  MOE_REQUIRE(T >= 0, MOE_EINVAL, "T = %lld < 0", (long long)T);
  MOE_REQUIRE(d > 0, MOE_EINVAL, "d = %d must be positive", d);
  MOE_REQUIRE(E >= 1, MOE_EINVAL, "E = %d must be >= 1", E);
  MOE_REQUIRE(k >= 1 && k <= E, MOE_EINVAL, "k = %d must satisfy 1 <= k <= E = %d", k, E);
  MOE_REQUIRE(E <= 256, MOE_EUNSUPPORTED, "E = %d > 256 is not supported", E);
  MOE_REQUIRE(k <= 16, MOE_EUNSUPPORTED, "k = %d > 16 is not supported", k);
  MOE_REQUIRE(d % 128 == 0, MOE_EUNSUPPORTED, "d = %d is not a multiple of 128", d);
  MOE_REQUIRE(T * (int64_t)k + T <= INT32_MAX, MOE_EUNSUPPORTED, "T*k too large for int32 indices");
  return MOE_OK;
}

int check_groups(int E, int k, int n_group, int topk_group) {
  if (n_group <= 1) return MOE_OK;
  MOE_REQUIRE(n_group <= 64 && E % n_group == 0, MOE_EINVAL,
              "n_group = %d must divide E = %d and be <= 64", n_group, E);
  MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, MOE_EINVAL,
              "topk_group = %d must be in [1, n_group = %d]", topk_group, n_group);
  MOE_REQUIRE(k <= topk_group * (E / n_group), MOE_EINVAL,
              "k = %d exceeds the %d experts of the chosen groups", k, topk_group * (E / n_group));
  return MOE_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  MOE_REQUIRE(have >= need, MOE_EWORKSPACE, "workspace of %zu bytes < required %zu", have, need);
  MOE_REQUIRE(need == 0 || ws != nullptr, MOE_EINVAL, "workspace pointer is NULL");
  MOE_REQUIRE(((uintptr_t)ws & 255) == 0, MOE_EINVAL, "workspace is not 256-byte aligned");
  return MOE_OK;
}

// Exact ceil(cf * N * k / E): cf is read as the shortest decimal that
// round-trips to the same double, i.e. M * 10^e with integer M.
int64_t exact_capacity(double cf, int64_t N, int k, int E) {
  char buf[64];
  int prec = 1;
  for (; prec <= 17; ++prec) {
    snprintf(buf, sizeof(buf), "%.*e", prec - 1, cf);
    if (strtod(buf, nullptr) == cf) break;
  }
  // buf = "D.DDDDe[+-]XX"
  unsigned long long M = 0;
  int ndig = 0;
  const char* p = buf;
  for (; *p && *p != 'e'; ++p)
    if (*p >= '0' && *p <= '9') { M = M * 10 + (unsigned)(*p - '0'); ++ndig; }
  const int e10 = atoi(p + 1) - (ndig - 1);
  typedef unsigned __int128 u128;
  u128 num = (u128)M * (u128)N * (u128)k;
  u128 den = (u128)E;
  if (e10 >= 0) {
    for (int i = 0; i < e10; ++i) num *= 10;
  } else {
    for (int i = 0; i < -e10; ++i) den *= 10;
  }
  const u128 c = (num + den - 1) / den;
  return (int64_t)c;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int64_t moe_capacity(double cf, int64_t N, int k, int E) {
  if (!(cf > 0.0) || !isfinite(cf)) return fail(MOE_EINVAL, "capacity factor must be finite and > 0");
  if (N < 0 || k < 1 || E < 1) return fail(MOE_EINVAL, "capacity needs N >= 0, k >= 1, E >= 1");
  const long double est = (long double)cf * (long double)N * (long double)k / (long double)E;
  if (est > 4.0e18L || cf > 1e15 || cf < 1e-15)
    return fail(MOE_EINVAL, "capacity factor %g out of range", cf);
  ok();
  return exact_capacity(cf, N, k, E);
}

// ------------------------------------------------------------------- route
size_t moe_route_workspace_size(int64_t T, int d, int E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return route_ws_bytes(T, d, E);
}

int check_backups(int k, int E, int n_backup, const int32_t* backup_ids, int64_t T) {
  const int most = k < E - k ? k : E - k;
  MOE_REQUIRE(n_backup >= 0 && n_backup <= most, MOE_EINVAL,
              "n_backup = %d must be in [0, min(k, E - k) = %d]", n_backup, most);
  MOE_REQUIRE(n_backup == 0 || T == 0 || backup_ids != nullptr, MOE_EINVAL, "NULL backup_ids");
  return MOE_OK;
}

int moe_route(const void* X, int dtype, int64_t T, int d, const void* Wg, int E,
              const float* bias, const float* logit_offset, int score, int k, int renorm,
              int n_group, int topk_group, float* logits, int32_t* topk_ids, float* topk_w,
              float* prob_sum, int n_backup, int32_t* backup_ids, void* ws, size_t ws_bytes,
              void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_router_dims(T, d, E, k))) return rc;
  if ((rc = check_groups(E, k, n_group, topk_group))) return rc;
  if ((rc = check_backups(k, E, n_backup, backup_ids, T))) return rc;
  MOE_REQUIRE(score == MOE_SOFTMAX || score == MOE_SIGMOID, MOE_EINVAL, "score %d unknown", score);
  MOE_REQUIRE(T == 0 || (X && Wg && topk_ids && topk_w), MOE_EINVAL, "NULL X, Wg, topk_ids or topk_w");
  MOE_REQUIRE(score == MOE_SIGMOID || bias == nullptr, MOE_EINVAL,
              "a selection bias is only defined for the sigmoid router");
  if ((rc = check_ws(ws, ws_bytes, route_ws_bytes(T, d, E)))) return rc;
  return hip_status(launch_route(X, dtype, T, d, Wg, E, bias, logit_offset, score, k, renorm,
                                 n_group, topk_group, logits, topk_ids, topk_w, prob_sum, ws,
                                 (hipStream_t)stream, nullptr, n_backup, backup_ids),
                    "moe_route");
}

// ------------------------------------------------------ expert-choice route
size_t moe_route_expert_choice_workspace_size(int64_t T, int d, int E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return route_ec_ws_bytes(T, d, E);
}

int moe_route_expert_choice(const void* X, int dtype, int64_t T, int d, const void* Wg, int E,
                            const float* logit_offset, int score, int64_t C, float* logits,
                            int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                            float* gates, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((rc = check_router_dims(T, d, E, 1))) return rc;
  MOE_REQUIRE(score == MOE_SOFTMAX || score == MOE_SIGMOID, MOE_EINVAL, "score %d unknown", score);
  MOE_REQUIRE(C >= 0, MOE_EINVAL, "C = %lld < 0", (long long)C);
  MOE_REQUIRE(T * (int64_t)E + T <= INT32_MAX, MOE_EUNSUPPORTED, "T*E too large for int32 indices");
  MOE_REQUIRE(offsets != nullptr, MOE_EINVAL, "NULL offsets");
  MOE_REQUIRE(T == 0 || (X && Wg && slot_row && gates), MOE_EINVAL,
              "NULL X, Wg, slot_row or gates");
  if ((rc = check_ws(ws, ws_bytes, route_ec_ws_bytes(T, d, E)))) return rc;
  const int Ce = (int)(C < T ? C : T);
  return hip_status(launch_route_ec(X, dtype, T, d, Wg, E, logit_offset, score, Ce, logits,
                                    offsets, nullptr, nullptr, sorted_slot, slot_row, gates,
                                    nullptr, 0, ws, (hipStream_t)stream),
                    "moe_route_expert_choice");
}

// ---------------------------------------------------------------- dispatch
size_t moe_dispatch_workspace_size(int64_t T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return dispatch_ws_bytes(T, k, E) + reroute_ws_bytes(T, k, E);
}

int moe_dispatch(const int32_t* topk_ids, int64_t T, int k, int E, int64_t capacity,
                 const int32_t* backup_ids, int n_backup, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slot, int32_t* slot_row, int32_t* n_kept, const void* X,
                 int dtype, int d, void* X_sorted, void* ws, size_t ws_bytes, void* stream) {
  MOE_REQUIRE(T >= 0, MOE_EINVAL, "T < 0");
  MOE_REQUIRE(E >= 1 && k >= 1 && k <= E, MOE_EINVAL, "need 1 <= k <= E");
  int rc0;
  if ((rc0 = check_backups(k, E, n_backup, backup_ids, T))) return rc0;
  MOE_REQUIRE(E <= 256, MOE_EUNSUPPORTED, "E = %d > 256 is not supported", E);
  MOE_REQUIRE(T * (int64_t)k <= INT32_MAX, MOE_EUNSUPPORTED, "T*k too large");
  MOE_REQUIRE(counts && offsets && n_kept, MOE_EINVAL, "NULL counts, offsets or n_kept");
  MOE_REQUIRE(T == 0 || (topk_ids && sorted_slot && slot_row), MOE_EINVAL,
              "NULL topk_ids, sorted_slot or slot_row");
  // A capacity of T*k or more never drops a slot; clamping it there keeps
  // every per-expert room and row count inside int32 in the kernels.
  const int64_t Tk = T * (int64_t)k;
  if (capacity > Tk) capacity = Tk > 0 ? Tk : 1;
  const bool gather = X_sorted != nullptr;
  if (gather) {
    int rc;
    if ((rc = check_dtype(dtype))) return rc;
    MOE_REQUIRE(X != nullptr, MOE_EINVAL, "X_sorted given without X");
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_EUNSUPPORTED, "d = %d is not a positive multiple of 128", d);
  }
  int rc;
  const size_t dws = dispatch_ws_bytes(T, k, E);
  if ((rc = check_ws(ws, ws_bytes, dws + reroute_ws_bytes(T, k, E)))) return rc;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_dispatch(topk_ids, T, k, E, capacity, 0, counts, offsets, sorted_slot,
                                 slot_row, n_kept, nullptr, ws, s);
  if (e == hipSuccess && capacity > 0 && n_backup > 0)
    e = launch_reroute(topk_ids, backup_ids, n_backup, T, k, E, capacity, 0, counts, offsets,
                       sorted_slot, slot_row, n_kept, nullptr, (char*)ws + dws, s);
  if (e == hipSuccess && gather)
    e = launch_gather(X, sorted_slot, n_kept, Tk, k, d, dtype == MOE_BF16 ? 2 : 4, X_sorted, s);
  return hip_status(e, "moe_dispatch");
}

// ------------------------------------------------------------- grouped FFN
size_t moe_grouped_ffn_workspace_size(int64_t max_rows, int G, int d, int F, int dtype) {
  if (max_rows < 0 || G < 1 || d <= 0 || F <= 0) return 0;
  return ffn_ws_bytes(max_rows, G, d, F, dtype);
}

int moe_grouped_ffn(const void* A, const int32_t* row_token, const int32_t* offsets, int G,
                    const void* W1, const void* W3, const void* W2, int dtype, int d, int F,
                    int64_t max_rows, float* Yrows, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  MOE_REQUIRE(G >= 1 && G <= 1024, MOE_EUNSUPPORTED, "G = %d must be in [1, 1024]", G);
  MOE_REQUIRE(max_rows >= 0 && max_rows <= INT32_MAX, MOE_EINVAL, "max_rows out of range");
  MOE_REQUIRE(d > 0 && F > 0, MOE_EINVAL, "d and F must be positive");
  MOE_REQUIRE(d % 128 == 0 && F % 128 == 0, MOE_EUNSUPPORTED,
              "d = %d and F = %d must be multiples of 128", d, F);
  MOE_REQUIRE(offsets != nullptr, MOE_EINVAL, "NULL offsets");
  MOE_REQUIRE(max_rows == 0 || (A && W1 && W3 && W2 && Yrows), MOE_EINVAL,
              "NULL A, W1, W3, W2 or Yrows");
  if ((rc = check_ws(ws, ws_bytes, ffn_ws_bytes(max_rows, G, d, F, dtype)))) return rc;
  // A holds max_rows rows when read directly; through row_token its row
  // count is not known here
  return hip_status(launch_grouped_ffn(A, row_token, offsets, G, W1, W3, W2, nullptr, nullptr,
                                       nullptr, -1, dtype, d, F, max_rows, Yrows, ws,
                                       (hipStream_t)stream, nullptr, row_token ? -1 : max_rows),
                    "moe_grouped_ffn");
}

int moe_grouped_ffn_fp8(const void* A, const int32_t* row_token, const int32_t* offsets, int G,
                        const uint8_t* W1, const uint8_t* W3, const uint8_t* W2,
                        const float* W1_scale, const float* W3_scale, const float* W2_scale,
                        int d, int F, int64_t max_rows, float* Yrows, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc;
  MOE_REQUIRE(G >= 1 && G <= 1024, MOE_EUNSUPPORTED, "G = %d must be in [1, 1024]", G);
  MOE_REQUIRE(max_rows >= 0 && max_rows <= INT32_MAX, MOE_EINVAL, "max_rows out of range");
  MOE_REQUIRE(d > 0 && F > 0, MOE_EINVAL, "d and F must be positive");
  MOE_REQUIRE(d % 128 == 0 && F % 128 == 0, MOE_EUNSUPPORTED,
              "d = %d and F = %d must be multiples of 128", d, F);
  MOE_REQUIRE(offsets != nullptr, MOE_EINVAL, "NULL offsets");
  MOE_REQUIRE(max_rows == 0 || (A && W1 && W3 && W2 && Yrows), MOE_EINVAL,
              "NULL A, W1, W3, W2 or Yrows");
  MOE_REQUIRE(max_rows == 0 || (W1_scale && W3_scale && W2_scale), MOE_EINVAL,
              "NULL weight scales");
  if ((rc = check_ws(ws, ws_bytes, ffn_ws_bytes(max_rows, G, d, F, MOE_BF16)))) return rc;
  const WeightScales q{W1_scale, W3_scale, W2_scale, nullptr, nullptr, nullptr};
  return hip_status(launch_grouped_ffn(A, row_token, offsets, G, W1, W3, W2, nullptr, nullptr,
                                       nullptr, -1, MOE_BF16, d, F, max_rows, Yrows, ws,
                                       (hipStream_t)stream, &q),
                    "moe_grouped_ffn_fp8");
}

// ----------------------------------------------------------------- combine
int moe_combine(const float* Yrows, const int32_t* slot_row, const float* topk_w, int64_t T,
                int k, int d, const float* shared, void* Y, int dtype, void* stream) {
  int rc;
  if ((rc = check_dtype(dtype))) return rc;
  MOE_REQUIRE(T >= 0 && k >= 1, MOE_EINVAL, "need T >= 0 and k >= 1");
  MOE_REQUIRE(k <= 256, MOE_EUNSUPPORTED, "k = %d > 256 is not supported", k);
  MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_EUNSUPPORTED, "d = %d is not a positive multiple of 128", d);
  MOE_REQUIRE(T * (int64_t)k <= INT32_MAX, MOE_EUNSUPPORTED, "T*k too large");
  MOE_REQUIRE(T == 0 || (Yrows && slot_row && topk_w && Y), MOE_EINVAL,
              "NULL Yrows, slot_row, topk_w or Y");
  return hip_status(launch_combine(Yrows, slot_row, topk_w, T, k, d, shared, nullptr, Y, dtype,
                                   (hipStream_t)stream),
                    "moe_combine");
}

int moe_bias_update(const int32_t* counts, int64_t T, int k, int E, float gamma, float* bias,
                    void* stream) {
  MOE_REQUIRE(T >= 0 && k >= 1 && E >= 1, MOE_EINVAL, "need T >= 0, k >= 1, E >= 1");
  MOE_REQUIRE(isfinite(gamma) && gamma >= 0.f, MOE_EINVAL, "gamma must be finite and >= 0");
  MOE_REQUIRE(counts && bias, MOE_EINVAL, "NULL counts or bias");
  MOE_REQUIRE(T * (int64_t)k <= INT32_MAX, MOE_EUNSUPPORTED, "T*k too large");
  return hip_status(launch_bias_update(counts, T, k, E, gamma, bias, (hipStream_t)stream),
                    "moe_bias_update");
}

int moe_balance(const int32_t* counts, const float* prob_sum, int64_t T, int k, int E, double* out,
                void* stream) {
  MOE_REQUIRE(counts && prob_sum && out, MOE_EINVAL, "NULL counts, prob_sum or out");
  MOE_REQUIRE(T >= 0 && k >= 1 && E >= 1, MOE_EINVAL, "need T >= 0, k >= 1, E >= 1");
  return hip_status(launch_balance(counts, prob_sum, T, k, E, out, (hipStream_t)stream),
                    "moe_balance");
}

// ----------------------------------------------------------------- forward
namespace {
struct FwdLayout {
  size_t route, ids, w, psum, counts, offsets, nkept, sorted, slotrow, rowtok, hist, ent, backup,
      rr, yrows, ffn, total;
};

// Backup experts per token for the overflow re-route: min(k, E - k) when
// the layer re-routes and has a capacity limit, else 0.
int layer_backups(const moe_layer* L) {
  if (!L->reroute || !(L->capacity_factor > 0) || L->routing != MOE_TOKEN_CHOICE) return 0;
  return L->k < L->E - L->k ? L->k : L->E - L->k;
}

bool expert_choice(const moe_layer* L) { return L->routing == MOE_EXPERT_CHOICE; }

// Tokens each expert takes under expert-choice routing: min(T, C) with
// C = ceil(cf * T * k / E), cf = 1 when no factor is set.  Factors outside
// moe_capacity's range give T (an upper bound; check_layer rejects them).
int64_t ec_capacity(const moe_layer* L, int64_t T) {
  const double cf = L->capacity_factor > 0 ? L->capacity_factor : 1.0;
  if (!(cf >= 1e-15 && cf <= 1e15)) return T;
  const long double est = (long double)cf * (long double)T * L->k / L->E;
  if (!(est < (long double)T)) return T;
  const int64_t c = exact_capacity(cf, T, L->k, L->E);
  return c < T ? c : T;
}

FwdLayout fwd_layout(const moe_layer* L, int64_t T) {
  FwdLayout o;
  const bool ec = expert_choice(L);
  const int64_t slots = T * (int64_t)(ec ? L->E : L->k);          // [T][k] or [T][E]
  const int64_t routed = ec ? L->E * ec_capacity(L, T) : T * (int64_t)L->k;
  const int64_t rows = routed + (L->n_shared ? T : 0);
  const int G = L->E + (L->n_shared ? 1 : 0);
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align256(bytes > 0 ? bytes : 1);
    return here;
  };
  o.route = take(ec ? route_ec_ws_bytes(T, L->d, L->E) : route_ws_bytes(T, L->d, L->E));
  o.ids = take((size_t)slots * 4);
  o.w = take((size_t)slots * 4);
  o.psum = take((size_t)L->E * 4);
  o.counts = take((size_t)L->E * 4);
  o.offsets = take((size_t)(L->E + 2) * 4);
  o.nkept = take(4);
  o.sorted = take((size_t)routed * 4);
  o.slotrow = take((size_t)slots * 4);
  o.rowtok = take((size_t)rows * 4);
  o.hist = take(dispatch_ws_bytes(T, L->k, L->E));
  o.ent = take((size_t)MOE_CEIL_DIV(T, 4) * 4);
  o.backup = take((size_t)T * layer_backups(L) * 4);
  o.rr = take(layer_backups(L) ? reroute_ws_bytes(T, L->k, L->E) : 0);
  o.yrows = take((size_t)rows * L->d * 4);
  o.ffn = take(ffn_ws_bytes(rows, G, L->d, L->F, L->dtype));
  o.total = at;
  return o;
}

int check_layer(const moe_layer* L, int64_t T) {
  MOE_REQUIRE(L != nullptr, MOE_EINVAL, "NULL layer");
  int rc;
  if ((rc = check_dtype(L->dtype))) return rc;
  if ((rc = check_router_dims(T, L->d, L->E, L->k))) return rc;
  MOE_REQUIRE(L->score == MOE_SOFTMAX || L->score == MOE_SIGMOID, MOE_EINVAL, "score %d unknown", L->score);
  MOE_REQUIRE(L->n_shared == 0 || L->n_shared == 1, MOE_EUNSUPPORTED, "n_shared must be 0 or 1");
  MOE_REQUIRE(L->F > 0 && L->F % 128 == 0, MOE_EUNSUPPORTED, "F = %d must be a positive multiple of 128", L->F);
  MOE_REQUIRE(L->Wg && L->W1 && L->W3 && L->W2, MOE_EINVAL, "NULL router or expert weights");
  MOE_REQUIRE(!L->n_shared || (L->Ws1 && L->Ws3 && L->Ws2), MOE_EINVAL, "NULL shared-expert weights");
  MOE_REQUIRE(L->score == MOE_SIGMOID || L->bias == nullptr, MOE_EINVAL,
              "a selection bias is only defined for the sigmoid router");
  MOE_REQUIRE(!(L->capacity_factor > 0) || isfinite(L->capacity_factor), MOE_EINVAL,
              "capacity factor must be finite");
  MOE_REQUIRE(L->wtype == MOE_W_DTYPE || L->wtype == MOE_W_FP8, MOE_EINVAL, "wtype %d unknown",
              L->wtype);
  if ((rc = check_groups(L->E, L->k, L->n_group, L->topk_group))) return rc;
  MOE_REQUIRE(L->routing == MOE_TOKEN_CHOICE || L->routing == MOE_EXPERT_CHOICE, MOE_EINVAL,
              "routing %d unknown", L->routing);
  MOE_REQUIRE(L->reroute == 0 || L->reroute == 1, MOE_EINVAL, "reroute must be 0 or 1");
  MOE_REQUIRE(!(L->reroute && L->routing == MOE_EXPERT_CHOICE), MOE_EINVAL,
              "the overflow re-route applies to top-k routing only");
  if (expert_choice(L)) {
    MOE_REQUIRE(!L->renorm && !L->bias && L->n_group <= 1, MOE_EINVAL,
                "expert-choice routing takes no renorm, bias or groups");
    MOE_REQUIRE(!(L->capacity_factor > 0) ||
                    (L->capacity_factor >= 1e-15 && L->capacity_factor <= 1e15),
                MOE_EINVAL, "capacity factor %g out of range", L->capacity_factor);
    MOE_REQUIRE(T * (int64_t)L->E + T <= INT32_MAX, MOE_EUNSUPPORTED,
                "T*E too large for int32 indices");
  }
  if (L->wtype == MOE_W_FP8) {
    MOE_REQUIRE(L->dtype == MOE_BF16, MOE_EUNSUPPORTED, "FP8 weights need a bf16 layer");
    MOE_REQUIRE(L->W1_scale && L->W3_scale && L->W2_scale, MOE_EINVAL, "NULL weight scales");
    MOE_REQUIRE(!L->n_shared || (L->Ws1_scale && L->Ws3_scale && L->Ws2_scale), MOE_EINVAL,
                "NULL shared-expert weight scales");
  }
  return MOE_OK;
}
}  // namespace

namespace {
// moe_forward with expert-choice routing: route and select in one step
// (offsets are e * C, known on the host), then the same grouped SwiGLU and
// a combine over the E slots of every token.
int forward_expert_choice(const moe_layer* L, const void* X, int64_t T, void* Y,
                          const moe_aux* aux, const FwdLayout& o, void* ws, void* stream) {
  moe_aux none;
  memset(&none, 0, sizeof(none));
  const moe_aux& a = aux ? *aux : none;
  MOE_REQUIRE(!a.topk_ids && !a.prob_sum && !a.balance && !a.health, MOE_EINVAL,
              "topk_ids, prob_sum, balance and health are top-k routing outputs; pass NULL "
              "with expert-choice routing");
  const int64_t C = ec_capacity(L, T);
  char* w = (char*)ws;
  auto pick = [&](void* user, size_t off) { return user ? user : (void*)(w + off); };
  float* gw = (float*)pick(a.topk_w, o.w);
  int32_t* offsets = (int32_t*)(w + o.offsets);            // E + 2 entries
  int32_t* nkept = (int32_t*)pick(a.n_kept, o.nkept);
  int32_t* slotrow = (int32_t*)pick(a.slot_row, o.slotrow);
  int32_t* rowtok = (int32_t*)(w + o.rowtok);
  float* yrows = (float*)pick(a.Yrows, o.yrows);
  hipStream_t s = (hipStream_t)stream;
  const int ns = L->n_shared ? 1 : 0;

  timing_mark("begin", s, 1);
  hipError_t e = launch_route_ec(X, L->dtype, T, L->d, L->Wg, L->E, L->logit_offset, L->score,
                                 (int)C, a.logits, offsets, a.counts, nkept, a.sorted_slot,
                                 slotrow, gw, rowtok, ns ? (int)T : 0, w + o.route, s);
  timing_mark("route", s);
  const WeightScales q{L->W1_scale, L->W3_scale, L->W2_scale, L->Ws1_scale, L->Ws3_scale,
                       L->Ws2_scale};
  if (e == hipSuccess)
    e = launch_grouped_ffn(X, rowtok, offsets, L->E + ns, L->W1, L->W3, L->W2, L->Ws1, L->Ws3,
                           L->Ws2, ns ? L->E : -1, L->dtype, L->d, L->F, L->E * C + ns * T,
                           yrows, w + o.ffn, s, L->wtype == MOE_W_FP8 ? &q : nullptr, T);
  if (e == hipSuccess)
    e = launch_combine(yrows, slotrow, gw, T, L->E, L->d, nullptr, ns ? nkept : nullptr, Y,
                       L->dtype, s);
  timing_mark("combine", s);
  if (e == hipSuccess && a.offsets)
    e = hipMemcpyAsync(a.offsets, offsets, (size_t)(L->E + 1) * 4, hipMemcpyDeviceToDevice, s);
  timing_mark("aux", s);
  return hip_status(e, "moe_forward");
}
}  // namespace

size_t moe_forward_workspace_size(const moe_layer* L, int64_t T) {
  if (!L || T < 0 || L->E < 1 || L->k < 1 || L->d <= 0 || L->F <= 0) return 0;
  return fwd_layout(L, T).total;
}

int moe_forward(const moe_layer* L, const void* X, int64_t T, void* Y, const moe_aux* aux,
                void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_layer(L, T))) return rc;
  MOE_REQUIRE(T == 0 || (X && Y), MOE_EINVAL, "NULL X or Y");
  const FwdLayout o = fwd_layout(L, T);
  if ((rc = check_ws(ws, ws_bytes, o.total))) return rc;
  if (expert_choice(L)) return forward_expert_choice(L, X, T, Y, aux, o, ws, stream);
  int64_t cap = 0;
  if (L->capacity_factor > 0) {
    cap = moe_capacity(L->capacity_factor, T, L->k, L->E);
    if (cap < 0) return (int)cap;
    // C >= T*k never drops a slot: clamped there, the kernels' per-expert
    // room and row counts stay inside int32
    const int64_t tk = T * (int64_t)L->k;
    if (cap > tk) cap = tk > 0 ? tk : 1;
  }
  moe_aux none;
  memset(&none, 0, sizeof(none));
  const moe_aux& a = aux ? *aux : none;
  char* w = (char*)ws;
  auto pick = [&](void* user, size_t off) { return user ? user : (void*)(w + off); };
  int32_t* ids = (int32_t*)pick(a.topk_ids, o.ids);
  float* gw = (float*)pick(a.topk_w, o.w);
  const bool need_ps = a.prob_sum || a.balance;
  float* psum = need_ps ? (float*)pick(a.prob_sum, o.psum) : nullptr;
  int32_t* counts = (int32_t*)pick(a.counts, o.counts);
  int32_t* offsets = (int32_t*)(w + o.offsets);            // E + 2 entries
  int32_t* nkept = (int32_t*)pick(a.n_kept, o.nkept);
  int32_t* sorted = (int32_t*)pick(a.sorted_slot, o.sorted);
  int32_t* slotrow = (int32_t*)pick(a.slot_row, o.slotrow);
  int32_t* rowtok = (int32_t*)(w + o.rowtok);
  float* yrows = (float*)pick(a.Yrows, o.yrows);
  hipStream_t s = (hipStream_t)stream;
  const int ns = L->n_shared ? 1 : 0;
  const int64_t Tk = T * (int64_t)L->k;

  timing_mark("begin", s, 1);
  float* ent = a.health ? (float*)(w + o.ent) : nullptr;
  const int nb = layer_backups(L);
  int32_t* backup = (int32_t*)(w + o.backup);
  hipError_t e = launch_route(X, L->dtype, T, L->d, L->Wg, L->E, L->bias, L->logit_offset,
                              L->score, L->k, L->renorm, L->n_group, L->topk_group, a.logits, ids,
                              gw, psum, w + o.route, s, ent, nb, backup);
  timing_mark("route", s);
  if (e == hipSuccess)
    e = launch_dispatch(ids, T, L->k, L->E, cap, ns ? (int)T : 0, counts, offsets, sorted, slotrow,
                        nkept, rowtok, w + o.hist, s);
  if (e == hipSuccess && nb > 0)
    e = launch_reroute(ids, backup, nb, T, L->k, L->E, cap, ns ? (int)T : 0, counts, offsets,
                       sorted, slotrow, nkept, rowtok, w + o.rr, s);
  timing_mark("dispatch", s);
  const WeightScales q{L->W1_scale, L->W3_scale, L->W2_scale, L->Ws1_scale, L->Ws3_scale,
                       L->Ws2_scale};
  if (e == hipSuccess)
    e = launch_grouped_ffn(X, rowtok, offsets, L->E + ns, L->W1, L->W3, L->W2, L->Ws1, L->Ws3,
                           L->Ws2, ns ? L->E : -1, L->dtype, L->d, L->F, Tk + ns * T, yrows,
                           w + o.ffn, s, L->wtype == MOE_W_FP8 ? &q : nullptr, T);
  if (e == hipSuccess)
    e = launch_combine(yrows, slotrow, gw, T, L->k, L->d, nullptr, ns ? nkept : nullptr, Y,
                       L->dtype, s);
  timing_mark("combine", s);
  if (e == hipSuccess && a.offsets)
    e = hipMemcpyAsync(a.offsets, offsets, (size_t)(L->E + 1) * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && a.balance) e = launch_balance(counts, psum, T, L->k, L->E, a.balance, s);
  if (e == hipSuccess && a.health)
    e = launch_router_health(counts, nkept, ent, T, L->k, L->E, a.health, s);
  timing_mark("aux", s);
  return hip_status(e, "moe_forward");
}

}  // extern "C"

// ------------------------------------------------- forward without allocation
// moe_forward's workspace taken from a fixed device array instead of the
// caller: for callers that cannot allocate.  Every GPU the library runs on
// holds its own copy of `scratch` until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch.
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on
// each device); MOE_OK or a negative status with the message set.
int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_EUNSUPPORTED,
              "device %d beyond the %d devices the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    MOE_REQUIRE(p != nullptr, MOE_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

size_t moe_forward_noalloc_max_bytes(void) { return kScratchBytes; }

int moe_forward_noalloc(const moe_layer* L, const void* X, int64_t T, void* Y,
                        const moe_aux* aux, void* stream) {
  int rc;
  if ((rc = check_layer(L, T))) return rc;
  const size_t need = fwd_layout(L, T).total;
  MOE_REQUIRE(need <= kScratchBytes, MOE_EWORKSPACE,
              "this layer and batch need %zu bytes of scratch, more than the %zu bytes "
              "moe_forward_noalloc holds; call moe_forward with a caller workspace",
              need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return moe_forward(L, X, T, Y, aux, ws, kScratchBytes, stream);
}

}  // extern "C"
