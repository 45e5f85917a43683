// C ABI of the library: host-side validation, workspace sizing and dispatch.
// Every argument is checked before any HIP call; no call allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "dsv4attn.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;

// Scratch of csa_index_topk_noalloc: one array per device, held until the process ends.
// In host code `scratch` is only a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress (per device, on the first call made with that device current).
constexpr size_t kScratchBytes = (size_t)48 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

dsv4_status fail(dsv4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsv4_status ok() {
  g_err[0] = '\0';
  return DSV4_OK;
}

// Device address of this device's scratch array (looked up once per device).
dsv4_status scratch_ptr(const char* what, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSV4_ERR_LAUNCH, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSV4_ERR_UNSUPPORTED, "%s: device %d out of range", what, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(DSV4_ERR_LAUNCH, "%s: hipGetSymbolAddress of the scratch array failed: %s", what,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DSV4_OK;
}

dsv4_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSV4_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Every size, count and stride argument is at most kMaxExtent, so that the products the
// validation and the launch plans form stay far inside int64_t; size_mul forms the ones
// that involve two caller-given sizes.
constexpr int64_t kMaxExtent = (int64_t)1 << 40;
bool extent_ok(std::initializer_list<int64_t> v) {
  for (int64_t x : v)
    if (x < 0 || x > kMaxExtent) return false;
  return true;
}
// a * b for non-negative sizes, or -1 when the product would exceed 2^62
int64_t size_mul(int64_t a, int64_t b) {
  if (a < 0 || b < 0) return -1;
  if (a != 0 && b > ((int64_t)1 << 62) / a) return -1;
  return a * b;
}

#define REQUIRE(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(DSV4_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define SUPPORT(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(DSV4_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

// Workspace protocol shared by the calls that need scratch memory:
//   workspace == NULL, ws_bytes != NULL : size query (writes *ws_bytes, launches nothing);
//   workspace == NULL, ws_bytes == NULL : run a call whose required size is 0;
//   workspace != NULL                   : run with *ws_bytes bytes of scratch.
dsv4_status workspace_check(const char* what, void* ws, size_t* ws_bytes, size_t need, bool* query) {
  *query = false;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    *query = true;
    return ok();
  }
  if (ws == nullptr) {
    if (need > 0) return fail(DSV4_ERR_WORKSPACE, "%s: requires a workspace of %zu bytes", what, need);
    return ok();
  }
  REQUIRE(ws_bytes != nullptr, "%s: ws_bytes must not be NULL when a workspace is given", what);
  if (*ws_bytes < need)
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu bytes required", what,
                *ws_bytes, need);
  return ok();
}

struct AttendCommon {
  const void *q, *kc, *vc, *kw, *vw;
  int dt;
  const int32_t *win_pos0, *q_pos;
  int64_t L;
  int32_t W;
  int64_t B, Q;
  int32_t H, D;
  int64_t N, kv_bstride, kv_rstride, w_rstride;
  float scale;
  void* out;
};

dsv4_status check_attend(const char* what, const AttendCommon& c) {
  REQUIRE(c.B >= 0 && c.Q >= 0 && c.N >= 0 && c.L >= 0 && c.W >= 0, "%s: sizes must be non-negative", what);
  REQUIRE(extent_ok({c.B, c.Q, c.N, c.L, c.kv_bstride, c.kv_rstride, c.w_rstride}),
          "%s: sizes and strides must lie in [0, 2^40]", what);
  REQUIRE(c.H > 0 && c.D > 0, "%s: H and D must be positive", what);
  SUPPORT(c.dt == DSV4_F32 || c.dt == DSV4_BF16, "%s: dt must be DSV4_F32 or DSV4_BF16", what);
  if (c.dt == DSV4_BF16) {
    SUPPORT(c.D == 128 || c.D == 256 || c.D == 512, "%s: bf16 path supports D in {128, 256, 512}, got %d", what, c.D);
    SUPPORT(c.H % 16 == 0 && c.H <= 64, "%s: bf16 path supports H in {16, 32, 48, 64}, got %d", what, c.H);
  } else {
    SUPPORT(c.D <= 512, "%s: f32 path supports D <= 512, got %d", what, c.D);
    SUPPORT(c.H <= 65535, "%s: H too large", what);
  }
  REQUIRE(c.kv_bstride == 0 || c.kv_bstride >= c.N, "%s: kv_bstride (%lld) must be 0 or >= N (%lld)", what,
          (long long)c.kv_bstride, (long long)c.N);
  REQUIRE(c.kv_rstride == 0 || c.kv_rstride >= c.D, "%s: kv_rstride (%lld) must be 0 or >= D (%d)", what,
          (long long)c.kv_rstride, c.D);
  REQUIRE(c.w_rstride == 0 || c.w_rstride >= c.D, "%s: w_rstride (%lld) must be 0 or >= D (%d)", what,
          (long long)c.w_rstride, c.D);
  if (c.dt == DSV4_BF16)
    REQUIRE(c.kv_rstride % 8 == 0 && c.w_rstride % 8 == 0, "%s: bf16 row strides must be multiples of 8", what);
  const int64_t BQ = size_mul(c.B, c.Q);
  REQUIRE(BQ >= 0 && BQ <= 65535, "%s: B*Q must be <= 65535", what);
  if (BQ > 0) {
    REQUIRE(c.q && c.out && c.q_pos, "%s: q, out and q_pos must not be NULL", what);
    REQUIRE(c.win_pos0 || c.W <= c.L, "%s: a ring window (win_pos0 == NULL) needs W (%d) <= L (%lld)", what, c.W,
            (long long)c.L);
    REQUIRE(c.N == 0 || (c.kc && c.vc), "%s: kc and vc must not be NULL when N > 0", what);
    REQUIRE(c.L == 0 || (c.kw && c.vw), "%s: kw and vw must not be NULL when L > 0", what);
  }
  REQUIRE(c.scale == c.scale, "%s: scale is NaN", what);
  return ok();
}

// csa_compress's checks of one pooling job, and its arguments for the launcher.
dsv4_status check_compress(const char* what, const void* x, int x_dt, const float* gate, const float* pos_bias,
                           int64_t B, int64_t T, int64_t C, int32_t m, int64_t x_bstride, void* y, uint8_t* y_scale,
                           int y_dt, int64_t y_bstride, dsv4::CompressArgs* out) {
  REQUIRE(B >= 0 && T >= 0 && C > 0, "%s: need B >= 0, T >= 0, C > 0", what);
  REQUIRE(extent_ok({B, T, C, x_bstride, y_bstride}), "%s: sizes and strides must lie in [0, 2^40]", what);
  REQUIRE(size_mul(B, T) >= 0 && size_mul(B, T) <= kMaxExtent, "%s: B*T must be <= 2^40", what);
  REQUIRE(m >= 1 && m <= 1024, "%s: m must be in [1, 1024], got %d", what, m);
  REQUIRE(T % m == 0, "%s: T (%lld) must be a multiple of m (%d)", what, (long long)T, m);
  SUPPORT(x_dt == DSV4_F32 || x_dt == DSV4_BF16, "%s: x_dt must be F32 or BF16", what);
  SUPPORT(y_dt >= DSV4_F32 && y_dt <= DSV4_FP8_KV, "%s: unknown y_dt %d", what, y_dt);
  if (y_dt == DSV4_FP8_KV)
    SUPPORT(C % 16 == 0 && C / 2 > dsv4::kFp8RopeDims, "%s: FP8 K|V rows need C %% 16 == 0 and C/2 > %d", what,
            dsv4::kFp8RopeDims);
  SUPPORT(C % 8 == 0, "%s: C must be a multiple of 8, got %lld", what, (long long)C);
  SUPPORT(C <= (x_dt == DSV4_F32 ? 1024 : 2048), "%s: C too large (f32: <= 1024, bf16: <= 2048)", what);
  if (y_dt == DSV4_MXFP4) SUPPORT(C % 32 == 0, "%s: MXFP4 output needs C %% 32 == 0", what);
  REQUIRE(x_bstride == 0 || x_bstride >= T, "%s: x_bstride must be 0 or >= T", what);
  REQUIRE(y_bstride == 0 || y_bstride >= T / m, "%s: y_bstride must be 0 or >= T/m", what);
  if (B * T > 0) {
    REQUIRE(x && gate && pos_bias && y, "%s: x, gate, pos_bias and y must not be NULL", what);
    if (y_dt == DSV4_MXFP4) REQUIRE(y_scale, "%s: y_scale must not be NULL for MXFP4 output", what);
  }
  dsv4::CompressArgs& a = *out;
  a.x = x; a.x_f32 = x_dt == DSV4_F32; a.gate = gate; a.bias = pos_bias;
  a.B = B; a.T = T; a.C = C; a.m = m;
  a.x_bs = x_bstride ? x_bstride : T;
  a.y_bs = y_bstride ? y_bstride : T / m;
  a.y = y; a.y_scale = y_scale; a.y_dt = y_dt;
  return ok();
}

dsv4::AttendArgs to_args(const AttendCommon& c, bool csa, const int32_t* idx, int k, int m, float* lse) {
  dsv4::AttendArgs a;
  a.csa = csa;
  a.q = c.q; a.kc = c.kc; a.vc = c.vc; a.f32 = c.dt == DSV4_F32;
  a.idx = idx; a.k = k; a.m = m;
  a.kw = c.kw; a.vw = c.vw; a.win_pos0 = c.win_pos0; a.L = c.L; a.W = c.W;
  a.q_pos = c.q_pos; a.B = c.B; a.Q = c.Q; a.H = c.H; a.D = c.D;
  a.N = c.N; a.kv_bs = c.kv_bstride ? c.kv_bstride : c.N;
  a.kv_rs = c.kv_rstride ? c.kv_rstride : c.D;
  a.w_rs = c.w_rstride ? c.w_rstride : c.D;
  a.scale = c.scale; a.out = c.out; a.lse = lse;
  return a;
}

// FP8 K/V rows (csa_attend_fp8kv / hca_attend_fp8kv): the shared checks with bf16 queries
// and outputs, then the row format, byte strides, alignment and scales.
struct Fp8Kv {
  int32_t d_rope;
  float k_scale, v_scale;
};
dsv4_status check_attend_fp8(const char* what, const AttendCommon& c, const Fp8Kv& f) {
  AttendCommon e = c;
  e.dt = DSV4_BF16;
  e.kv_rstride = 0;   // byte strides, checked below
  e.w_rstride = 0;
  dsv4_status s = check_attend(what, e);
  if (s != DSV4_OK) return s;
  SUPPORT(c.D == 512, "%s: FP8 K/V rows support D = 512, got %d", what, c.D);
  SUPPORT(f.d_rope == dsv4::kFp8RopeDims, "%s: FP8 K/V rows support d_rope = %d, got %d", what,
          dsv4::kFp8RopeDims, f.d_rope);
  const int64_t kb = c.D + f.d_rope;   // bytes of a K row (codes + bf16 dims)
  REQUIRE(c.kv_rstride == 0 || (c.kv_rstride >= kb && c.kv_rstride % 16 == 0),
          "%s: kv_rstride (%lld bytes) must be 0 or a multiple of 16 that is >= %lld", what,
          (long long)c.kv_rstride, (long long)kb);
  REQUIRE(c.w_rstride == 0 || (c.w_rstride >= kb && c.w_rstride % 16 == 0),
          "%s: w_rstride (%lld bytes) must be 0 or a multiple of 16 that is >= %lld", what, (long long)c.w_rstride,
          (long long)kb);
  for (const void* p : {c.kc, c.vc, c.kw, c.vw})
    REQUIRE(((uintptr_t)p & 15) == 0, "%s: kc, vc, kw and vw must be 16-byte aligned", what);
  REQUIRE(f.k_scale == f.k_scale && f.v_scale == f.v_scale && f.k_scale - f.k_scale == 0.f &&
              f.v_scale - f.v_scale == 0.f,
          "%s: k_scale and v_scale must be finite", what);
  return ok();
}

void to_args_fp8(dsv4::AttendArgs& a, const AttendCommon& c, const Fp8Kv& f) {
  a.f8 = true;
  a.k_scale = f.k_scale;
  a.v_scale = f.v_scale;
  const int64_t kb = c.D + f.d_rope;
  a.kv_rs = c.kv_rstride ? c.kv_rstride : kb;
  a.v_rs = c.kv_rstride ? c.kv_rstride : c.D;
  a.w_rs = c.w_rstride ? c.w_rstride : kb;
  a.wv_rs = c.w_rstride ? c.w_rstride : c.D;
}

dsv4_status run_attend(const char* what, const dsv4::AttendArgs& a, void* ws, size_t* ws_bytes, hipStream_t st) {
  dsv4::AttendPlan p = dsv4::plan_attend(a);
  if (!p.supported)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: the key list (k or N plus the window) needs more than 1024 splits "
                "of the longest supported chunk; use a smaller window W", what);
  bool query;
  dsv4_status s = workspace_check(what, ws, ws_bytes, p.ws_bytes, &query);
  if (s != DSV4_OK || query) return s;
  return launched(dsv4::launch_attend(a, p, ws, st), what);
}

}  // namespace

namespace dsv4 {
bool take_kernel_timing(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_time_start) return false;
  *start = g_time_start;
  *stop = g_time_stop;
  g_time_start = g_time_stop = nullptr;
  return true;
}
}  // namespace dsv4

extern "C" {

dsv4_status dsv4_time_next_kernel(hipEvent_t start, hipEvent_t stop) {
  REQUIRE((start == nullptr) == (stop == nullptr), "dsv4_time_next_kernel: give both events or neither");
  g_time_start = start;
  g_time_stop = stop;
  return ok();
}

int dsv4_version(void) { return 100; }

dsv4_status dsv4_debug_flags(uint32_t* flags) {
  REQUIRE(flags != nullptr, "dsv4_debug_flags: flags must not be NULL");
  *flags = 0;
#ifdef DSV4_DEBUG
  *flags = dsv4::debug_flags_attend() | dsv4::debug_flags_index() | dsv4::debug_flags_compress();
  return ok();
#else
  return fail(DSV4_ERR_UNSUPPORTED, "dsv4_debug_flags: this library was built without DSV4_DEBUG");
#endif
}

const char* dsv4_status_string(int s) {
  switch (s) {
    case DSV4_OK: return "DSV4_OK";
    case DSV4_ERR_INVALID_ARG: return "DSV4_ERR_INVALID_ARG";
    case DSV4_ERR_UNSUPPORTED: return "DSV4_ERR_UNSUPPORTED";
    case DSV4_ERR_WORKSPACE: return "DSV4_ERR_WORKSPACE";
    case DSV4_ERR_LAUNCH: return "DSV4_ERR_LAUNCH";
    default: return "DSV4_ERR_UNKNOWN";
  }
}

const char* dsv4_last_error(void) { return g_err; }

dsv4_status csa_compress(const void* x, int x_dt, const float* gate, const float* pos_bias, int64_t B, int64_t T,
                         int64_t C, int32_t m, int64_t x_bstride, void* y, uint8_t* y_scale, int y_dt,
                         int64_t y_bstride, hipStream_t stream) {
  const char* what = "csa_compress";
  dsv4::CompressArgs a;
  dsv4_status s = check_compress(what, x, x_dt, gate, pos_bias, B, T, C, m, x_bstride, y, y_scale, y_dt, y_bstride, &a);
  if (s != DSV4_OK) return s;
  if (a.total_blocks() == 0) return ok();
  return launched(dsv4::launch_compress(a, stream), what);
}

dsv4_status csa_compress2(const void* x, const void* x2, int x_dt, const float* gate, const float* pos_bias,
                          int64_t B, int64_t T, int32_t m, int64_t C, int64_t x_bstride, void* y, uint8_t* y_scale,
                          int y_dt, int64_t y_bstride, int64_t C2, int64_t x2_bstride, void* y2, uint8_t* y2_scale,
                          int y2_dt, int64_t y2_bstride, hipStream_t stream) {
  const char* what = "csa_compress2";
  dsv4::CompressArgs a, b;
  dsv4_status s = check_compress(what, x, x_dt, gate, pos_bias, B, T, C, m, x_bstride, y, y_scale, y_dt, y_bstride, &a);
  if (s != DSV4_OK) return s;
  s = check_compress(what, x2, x_dt, gate, pos_bias, B, T, C2, m, x2_bstride, y2, y2_scale, y2_dt, y2_bstride, &b);
  if (s != DSV4_OK) return s;
  SUPPORT(x_dt == DSV4_BF16 && (y_dt == DSV4_BF16 || y_dt == DSV4_FP8_KV) && y2_dt == DSV4_MXFP4,
          "%s: supports bf16 x with (y_dt, y2_dt) = (BF16 or FP8_KV, MXFP4)", what);
  if (a.total_blocks() == 0) return ok();
  return launched(dsv4::launch_compress2(a, b, stream), what);
}

dsv4_status kv_cache_append(const void* x_new, int x_dt, const float* gate_new, const int32_t* pos, int64_t B,
                            int64_t C, void* win, float* win_gate, int64_t L, const float* pos_bias, int32_t m,
                            void* y, uint8_t* y_scale, int y_dt, int64_t N, int64_t y_bstride, hipStream_t stream) {
  const char* what = "kv_cache_append";
  REQUIRE(B >= 0 && C > 0 && N >= 0, "%s: need B >= 0, C > 0, N >= 0", what);
  REQUIRE(extent_ok({B, C, N, L, y_bstride}), "%s: sizes and strides must lie in [0, 2^40]", what);
  REQUIRE(m >= 1 && m <= 1024, "%s: m must be in [1, 1024], got %d", what, m);
  SUPPORT(x_dt == DSV4_F32 || x_dt == DSV4_BF16, "%s: x_dt must be F32 or BF16", what);
  SUPPORT(y_dt >= DSV4_F32 && y_dt <= DSV4_FP8_KV, "%s: unknown y_dt %d", what, y_dt);
  if (y_dt == DSV4_FP8_KV)
    SUPPORT(C % 16 == 0 && C / 2 > dsv4::kFp8RopeDims, "%s: FP8 K|V rows need C %% 16 == 0 and C/2 > %d", what,
            dsv4::kFp8RopeDims);
  SUPPORT(C % 8 == 0, "%s: C must be a multiple of 8, got %lld", what, (long long)C);
  SUPPORT(C <= (x_dt == DSV4_F32 ? 1024 : 2048), "%s: C too large (f32: <= 1024, bf16: <= 2048)", what);
  if (y_dt == DSV4_MXFP4) SUPPORT(C % 32 == 0, "%s: MXFP4 output needs C %% 32 == 0", what);
  REQUIRE(L >= m && L % m == 0, "%s: L (%lld) must be a positive multiple of m (%d)", what, (long long)L, m);
  REQUIRE(y_bstride == 0 || y_bstride >= N, "%s: y_bstride must be 0 or >= N", what);
  REQUIRE(B <= 65535, "%s: B must be <= 65535", what);
  if (B > 0) {
    REQUIRE(x_new && gate_new && pos && win && win_gate && pos_bias,
            "%s: x_new, gate_new, pos, win, win_gate and pos_bias must not be NULL", what);
    REQUIRE(N == 0 || y, "%s: y must not be NULL when N > 0", what);
    if (y_dt == DSV4_MXFP4 && N > 0) REQUIRE(y_scale, "%s: y_scale must not be NULL for MXFP4 output", what);
  }
  dsv4::AppendArgs a;
  a.x_new = x_new; a.x_f32 = x_dt == DSV4_F32; a.gate_new = gate_new; a.pos = pos;
  a.win = win; a.win_gate = win_gate;
  a.B = B; a.L = L; a.C = C; a.bias = pos_bias; a.m = m;
  a.y = y; a.y_scale = y_scale; a.y_dt = y_dt; a.y_bs = y_bstride ? y_bstride : N; a.N = N;
  if (B == 0) return ok();
  return launched(dsv4::launch_append(a, stream), what);
}

}  // extern "C"

namespace {

// csa_index_topk and its allocation-free variant.  noalloc: the workspace is the
// library's static scratch array of this device (workspace and ws_bytes are ignored).
dsv4_status index_topk_impl(const char* what, const void* qi, int qi_dt, const float* wi, const void* ki,
                            const uint8_t* ki_scale, int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q,
                            int32_t HI, int32_t DI, int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                            int32_t* out_idx, float* out_score, void* workspace, size_t* ws_bytes,
                            hipStream_t stream, bool noalloc, const dsv4_block_pool* pool = nullptr) {
  REQUIRE(B >= 0 && Q >= 0 && N >= 0, "%s: sizes must be non-negative", what);
  REQUIRE(extent_ok({B, Q, N, ki_bstride}), "%s: sizes and strides must lie in [0, 2^40]", what);
  REQUIRE(m >= 1, "%s: m must be >= 1", what);
  REQUIRE(k >= 1 && k <= 4096, "%s: k must be in [1, 4096], got %d", what, k);
  REQUIRE(N < (int64_t)1 << 31, "%s: N must be < 2^31", what);
  REQUIRE(ki_bstride == 0 || ki_bstride >= N, "%s: ki_bstride must be 0 or >= N", what);
  REQUIRE(size_mul(B, Q) >= 0 && size_mul(B, Q) <= 65535, "%s: B*Q must be <= 65535", what);
  int kind;
  if (qi_dt == DSV4_F32 && ki_dt == DSV4_F32) kind = dsv4::KEY_F32;
  else if (qi_dt == DSV4_BF16 && ki_dt == DSV4_BF16) kind = dsv4::KEY_BF16;
  else if (qi_dt == DSV4_BF16 && ki_dt == DSV4_MXFP4) kind = dsv4::KEY_MXFP4;
  else if (qi_dt == DSV4_FP8_E4M3 && ki_dt == DSV4_FP8_E4M3) kind = dsv4::KEY_FP8;
  else if (qi_dt == DSV4_MXFP4 && ki_dt == DSV4_MXFP4) kind = dsv4::KEY_MXFP4_Q4;
  else return fail(DSV4_ERR_UNSUPPORTED, "%s: unsupported (qi_dt, ki_dt) = (%d, %d)", what, qi_dt, ki_dt);
  if (kind == dsv4::KEY_F32) {
    SUPPORT(HI >= 1 && HI <= 16, "%s: f32 path supports HI in [1, 16], got %d", what, HI);
    SUPPORT(DI >= 1 && DI <= 256, "%s: f32 path supports DI in [1, 256], got %d", what, DI);
  } else {
    SUPPORT(HI == 4 || HI == 8 || HI == 16, "%s: HI must be 4, 8 or 16, got %d", what, HI);
    SUPPORT(DI == 32 || DI == 64 || DI == 128 || DI == 256, "%s: DI must be 32, 64, 128 or 256, got %d", what, DI);
    if (kind == dsv4::KEY_MXFP4_Q4)
      SUPPORT(DI == 128 || DI == 256, "%s: MXFP4 queries need DI of 128 or 256, got %d", what, DI);
  }
  const int64_t R = B * Q;
  if (R > 0) {
    REQUIRE(qi && wi && q_pos && out_idx, "%s: qi, wi, q_pos and out_idx must not be NULL", what);
    REQUIRE(N == 0 || ki, "%s: ki must not be NULL when N > 0", what);
    if (kind == dsv4::KEY_MXFP4 || kind == dsv4::KEY_MXFP4_Q4)
      REQUIRE(N == 0 || ki_scale, "%s: ki_scale must not be NULL for MXFP4", what);
  }
  dsv4::IndexArgs a;
  a.qi = qi; a.wi = wi; a.ki = ki; a.ki_scale = ki_scale; a.kind = kind; a.q_pos = q_pos;
  // MXFP4 queries: the scale bytes follow the codes in the same allocation
  a.qi_scale = kind == dsv4::KEY_MXFP4_Q4 ? reinterpret_cast<const uint8_t*>(qi) + R * HI * (DI / 2) : nullptr;
  a.B = B; a.Q = Q; a.HI = HI; a.DI = DI; a.N = N; a.k_bs = ki_bstride ? ki_bstride : N;
  a.m = m; a.k = k; a.out_idx = out_idx; a.out_score = out_score;
  if (pool) {
    // the newest block of each sequence, pooled as csa_compress2 would into row pool->row
    SUPPORT(ki_dt == DSV4_MXFP4, "%s: the pooled indexer keys are MXFP4 (ki_dt must be DSV4_MXFP4)", what);
    SUPPORT((int64_t)m * DI <= 512, "%s: m * DI must be <= 512 (the key is pooled by one wave)", what);
    SUPPORT(m >= 1 && (m & (m - 1)) == 0,
            "%s: m must be a power of two (the key's rows combine inside one wave), got %d", what, m);
    REQUIRE(pool->row >= 0 && pool->row < N, "%s: pool->row (%lld) must lie in [0, N)", what, (long long)pool->row);
    SUPPORT(pool->y_dt == DSV4_BF16 || pool->y_dt == DSV4_FP8_KV, "%s: pool->y_dt must be DSV4_BF16 or DSV4_FP8_KV",
            what);
    REQUIRE(pool->y_bstride == 0 || pool->y_bstride > pool->row,
            "%s: pool->y_bstride must be 0 or more than pool->row", what);
    dsv4::CompressArgs ca, cb;
    const int64_t y_bs = pool->y_bstride ? pool->y_bstride : N;
    dsv4_status ps = check_compress(what, pool->x, DSV4_BF16, pool->gate, pool->pos_bias, B, m, pool->C, m,
                                    pool->x_bstride, pool->y, pool->y_scale, pool->y_dt, y_bs, &ca);
    if (ps != DSV4_OK) return ps;
    uint8_t* krow = ki ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(ki)) + pool->row * (DI / 2) : nullptr;
    uint8_t* srow = ki_scale ? const_cast<uint8_t*>(ki_scale) + pool->row * (DI / 32) : nullptr;
    ps = check_compress(what, pool->x2, DSV4_BF16, pool->gate, pool->pos_bias, B, m, DI, m, pool->x2_bstride, krow,
                        srow, DSV4_MXFP4, a.k_bs, &cb);
    if (ps != DSV4_OK) return ps;
    dsv4::IndexPool& ip = a.pool;
    ip.on = B > 0;
    ip.x = pool->x; ip.x2 = pool->x2; ip.gate = pool->gate; ip.bias = pool->pos_bias;
    ip.x_bs = ca.x_bs; ip.x2_bs = cb.x_bs; ip.C = pool->C;
    ip.y = pool->y; ip.y_scale = pool->y_scale; ip.y_dt = pool->y_dt; ip.y_bs = y_bs; ip.row = pool->row;
  }
  const size_t need = dsv4::topk_workspace_bytes(a);
  size_t scratch_size = 0;
  if (noalloc) {
    if (need > kScratchBytes)
      return fail(DSV4_ERR_UNSUPPORTED, "%s: this call needs %zu bytes of scratch, more than the %zu bytes of the "
                  "static scratch array; use csa_index_topk with a workspace", what, need, kScratchBytes);
    if (R == 0) return ok();
    dsv4_status st = scratch_ptr(what, &workspace);
    if (st != DSV4_OK) return st;
    scratch_size = kScratchBytes;
    ws_bytes = &scratch_size;
  }
  bool query;
  dsv4_status s = workspace_check(what, workspace, ws_bytes, need, &query);
  if (s != DSV4_OK || query || R == 0) return s;
  return launched(dsv4::launch_index_topk(a, workspace, stream), what);
}

}  // namespace

extern "C" {

dsv4_status csa_index_topk(const void* qi, int qi_dt, const float* wi, const void* ki, const uint8_t* ki_scale,
                           int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q, int32_t HI, int32_t DI, int64_t N,
                           int64_t ki_bstride, int32_t m, int32_t k, int32_t* out_idx, float* out_score,
                           void* workspace, size_t* ws_bytes, hipStream_t stream) {
  return index_topk_impl("csa_index_topk", qi, qi_dt, wi, ki, ki_scale, ki_dt, q_pos, B, Q, HI, DI, N, ki_bstride, m,
                         k, out_idx, out_score, workspace, ws_bytes, stream, false);
}

dsv4_status csa_pool_index_topk(const dsv4_block_pool* pool, const void* qi, int qi_dt, const float* wi, void* ki,
                                uint8_t* ki_scale, int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q,
                                int32_t HI, int32_t DI, int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                                int32_t* out_idx, float* out_score, void* workspace, size_t* ws_bytes,
                                hipStream_t stream) {
  REQUIRE(pool != nullptr, "csa_pool_index_topk: pool must not be NULL");
  return index_topk_impl("csa_pool_index_topk", qi, qi_dt, wi, ki, ki_scale, ki_dt, q_pos, B, Q, HI, DI, N,
                         ki_bstride, m, k, out_idx, out_score, workspace, ws_bytes, stream, false, pool);
}

dsv4_status csa_index_topk_noalloc(const void* qi, int qi_dt, const float* wi, const void* ki,
                                   const uint8_t* ki_scale, int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q,
                                   int32_t HI, int32_t DI, int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                                   int32_t* out_idx, float* out_score, hipStream_t stream) {
  return index_topk_impl("csa_index_topk_noalloc", qi, qi_dt, wi, ki, ki_scale, ki_dt, q_pos, B, Q, HI, DI, N,
                         ki_bstride, m, k, out_idx, out_score, nullptr, nullptr, stream, true);
}

dsv4_status csa_attend(const void* q, const void* kc, const void* vc, int dt, const int32_t* idx, int32_t k,
                       const void* kw, const void* vw, const int32_t* win_pos0, int64_t L, int32_t W,
                       const int32_t* q_pos, int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N,
                       int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float scale, void* out, float* lse,
                       void* workspace, size_t* ws_bytes, hipStream_t stream) {
  const char* what = "csa_attend";
  AttendCommon c{q, kc, vc, kw, vw, dt, win_pos0, q_pos, L, W, B, Q, H, D, N, kv_bstride, kv_rstride, w_rstride,
                 scale, out};
  dsv4_status s = check_attend(what, c);
  if (s != DSV4_OK) return s;
  REQUIRE(k >= 0 && k <= 65536, "%s: k must be in [0, 65536]", what);
  if (B * Q > 0 && k > 0) REQUIRE(idx, "%s: idx must not be NULL", what);
  return run_attend(what, to_args(c, true, idx, k, 1, lse), workspace, ws_bytes, stream);
}

dsv4_status hca_attend(const void* q, const void* kc, const void* vc, int dt, int32_t m, const void* kw,
                       const void* vw, const int32_t* win_pos0, int64_t L, int32_t W, const int32_t* q_pos,
                       int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int64_t kv_bstride,
                       int64_t kv_rstride, int64_t w_rstride, float scale, void* out, float* lse, void* workspace,
                       size_t* ws_bytes, hipStream_t stream) {
  const char* what = "hca_attend";
  AttendCommon c{q, kc, vc, kw, vw, dt, win_pos0, q_pos, L, W, B, Q, H, D, N, kv_bstride, kv_rstride, w_rstride,
                 scale, out};
  dsv4_status s = check_attend(what, c);
  if (s != DSV4_OK) return s;
  REQUIRE(m >= 1, "%s: m must be >= 1", what);
  return run_attend(what, to_args(c, false, nullptr, 0, m, lse), workspace, ws_bytes, stream);
}

dsv4_status hca_pool_attend(const void* x, const float* gate, const float* pos_bias, int64_t x_bstride,
                            const void* q, const void* kc, const void* vc, int dt, int32_t m, const void* kw,
                            const void* vw, const int32_t* win_pos0, int64_t L, int32_t W, const int32_t* q_pos,
                            int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int64_t kv_bstride,
                            int64_t kv_rstride, int64_t w_rstride, float scale, void* out, float* lse, void* workspace,
                            size_t* ws_bytes, hipStream_t stream) {
  const char* what = "hca_pool_attend";
  AttendCommon c{q, kc, vc, kw, vw, dt, win_pos0, q_pos, L, W, B, Q, H, D, N, kv_bstride, kv_rstride, w_rstride,
                 scale, out};
  dsv4_status s = check_attend(what, c);
  if (s != DSV4_OK) return s;
  REQUIRE(m >= 1 && m <= 1024, "%s: m must be in [1, 1024], got %d", what, m);
  SUPPORT(dt == DSV4_BF16 && D == 512, "%s: supports bf16 with D = 512", what);
  SUPPORT(Q < 16, "%s: supports fewer than 16 queries per sequence (decode)", what);
  REQUIRE(N >= 1, "%s: N must be >= 1 (the pooled block becomes entry N - 1)", what);
  const int64_t rs = kv_rstride ? kv_rstride : D;
  REQUIRE(B == 0 || (kc && vc && reinterpret_cast<const uint16_t*>(vc) == reinterpret_cast<const uint16_t*>(kc) + D &&
                     rs >= 2 * D),
          "%s: K and V rows must sit side by side in one buffer (vc = kc + D, kv_rstride >= 2D)", what);
  REQUIRE(extent_ok({x_bstride}) && (x_bstride == 0 || x_bstride >= m), "%s: x_bstride must be 0 or >= m", what);
  if (B * Q > 0) REQUIRE(x && gate && pos_bias, "%s: x, gate and pos_bias must not be NULL", what);
  AttendCommon cn = c;
  cn.N = N - 1;                                    // the splits stop before the pooled entry
  cn.kv_bstride = kv_bstride ? kv_bstride : N;
  dsv4::AttendArgs a = to_args(cn, false, nullptr, 0, m, lse);
  a.pool.on = B * Q > 0;
  a.pool.x = x;
  a.pool.gate = gate;
  a.pool.bias = pos_bias;
  a.pool.x_bs = x_bstride ? x_bstride : m;
  a.pool.row = N - 1;
  return run_attend(what, a, workspace, ws_bytes, stream);
}

dsv4_status csa_attend_fp8kv(const void* q, const void* kc, const void* vc, const int32_t* idx, int32_t k,
                             const void* kw, const void* vw, const int32_t* win_pos0, int64_t L, int32_t W,
                             const int32_t* q_pos, int64_t B, int64_t Q, int32_t H, int32_t D, int32_t d_rope,
                             int64_t N, int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float k_scale,
                             float v_scale, float scale, void* out, float* lse, void* workspace, size_t* ws_bytes,
                             hipStream_t stream) {
  const char* what = "csa_attend_fp8kv";
  AttendCommon c{q, kc, vc, kw, vw, DSV4_BF16, win_pos0, q_pos, L, W, B, Q, H, D, N, kv_bstride, kv_rstride,
                 w_rstride, scale, out};
  const Fp8Kv f{d_rope, k_scale, v_scale};
  dsv4_status s = check_attend_fp8(what, c, f);
  if (s != DSV4_OK) return s;
  REQUIRE(k >= 0 && k <= 65536, "%s: k must be in [0, 65536]", what);
  if (B * Q > 0 && k > 0) REQUIRE(idx, "%s: idx must not be NULL", what);
  dsv4::AttendArgs a = to_args(c, true, idx, k, 1, lse);
  to_args_fp8(a, c, f);
  return run_attend(what, a, workspace, ws_bytes, stream);
}

dsv4_status hca_attend_fp8kv(const void* q, const void* kc, const void* vc, int32_t m, const void* kw, const void* vw,
                             const int32_t* win_pos0, int64_t L, int32_t W, const int32_t* q_pos, int64_t B,
                             int64_t Q, int32_t H, int32_t D, int32_t d_rope, int64_t N, int64_t kv_bstride,
                             int64_t kv_rstride, int64_t w_rstride, float k_scale, float v_scale, float scale,
                             void* out, float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream) {
  const char* what = "hca_attend_fp8kv";
  AttendCommon c{q, kc, vc, kw, vw, DSV4_BF16, win_pos0, q_pos, L, W, B, Q, H, D, N, kv_bstride, kv_rstride,
                 w_rstride, scale, out};
  const Fp8Kv f{d_rope, k_scale, v_scale};
  dsv4_status s = check_attend_fp8(what, c, f);
  if (s != DSV4_OK) return s;
  REQUIRE(m >= 1, "%s: m must be >= 1", what);
  dsv4::AttendArgs a = to_args(c, false, nullptr, 0, m, lse);
  to_args_fp8(a, c, f);
  return run_attend(what, a, workspace, ws_bytes, stream);
}

dsv4_status lse_merge(const float* o_parts, const float* lse_parts, int32_t P, int64_t R, int32_t D, void* out,
                      int out_dt, float* lse_out, hipStream_t stream) {
  const char* what = "lse_merge";
  REQUIRE(P >= 1 && P <= 1024, "%s: P must be in [1, 1024], got %d", what, P);
  REQUIRE(R >= 0, "%s: R must be non-negative", what);
  REQUIRE(D > 0 && D % 4 == 0 && D <= 4096, "%s: D must be a positive multiple of 4, <= 4096", what);
  SUPPORT(out_dt == DSV4_F32 || out_dt == DSV4_BF16, "%s: out_dt must be F32 or BF16", what);
  REQUIRE(R <= 0x7fffffff, "%s: R too large", what);
  if (R > 0) REQUIRE(o_parts && lse_parts && out, "%s: o_parts, lse_parts and out must not be NULL", what);
  if (R == 0) return ok();
  return launched(dsv4::launch_lse_merge(o_parts, lse_parts, P, R, D, out, out_dt == DSV4_F32, lse_out, stream),
                  what);
}

}  // extern "C"
