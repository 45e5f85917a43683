// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsv4 {

// Events armed by dsv4_time_next_kernel() on this thread, consumed by the next main
// kernel launch (false when nothing is armed).
bool take_kernel_timing(hipEvent_t* start, hipEvent_t* stop);

// Launch of a call's main kernel: recorded between the armed events when there are any.
#define DSV4_LAUNCH_MAIN(kernel, grid, block, smem, stream, ...)                                     \
  do {                                                                                             \
    hipEvent_t dsv4_t0_, dsv4_t1_;                                                                 \
    if (::dsv4::take_kernel_timing(&dsv4_t0_, &dsv4_t1_))                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, smem, stream, dsv4_t0_, dsv4_t1_, 0, __VA_ARGS__);  \
    else                                                                                           \
      hipLaunchKernelGGL(kernel, grid, block, smem, stream, __VA_ARGS__);                          \
  } while (0)

struct CompressArgs {
  const void* x;
  bool x_f32;
  const float* gate;
  const float* bias;
  int64_t B, T, C;
  int m;
  int64_t x_bs, y_bs;   // batch strides in rows
  void* y;
  uint8_t* y_scale;
  int y_dt;             // 0 f32, 1 bf16, 2 fp8 e4m3, 3 MXFP4, 4 FP8 K|V rows
  int64_t total_blocks() const { return B * (T / m); }
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);
// two jobs with the same gate, bias, B, T and m in one launch; bf16 x, (y_dt, y2_dt) in
// {(BF16, MXFP4), (FP8_KV, MXFP4)}
hipError_t launch_compress2(const CompressArgs& a, const CompressArgs& b, hipStream_t st);

struct AppendArgs {
  const void* x_new;
  bool x_f32;
  const float* gate_new;
  const int32_t* pos;
  void* win;
  float* win_gate;
  int64_t B, L, C;
  const float* bias;
  int m;
  void* y;
  uint8_t* y_scale;
  int y_dt;             // 0 f32, 1 bf16, 2 fp8 e4m3, 3 MXFP4, 4 FP8 K|V rows
  int64_t y_bs, N;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

// ---------------------------------------------------------------- indexer + top-k
// KEY_MXFP4: bf16 queries x MXFP4 keys; KEY_MXFP4_Q4: MXFP4 queries x MXFP4 keys
enum KeyKind { KEY_F32 = 0, KEY_BF16 = 1, KEY_FP8 = 2, KEY_MXFP4 = 3, KEY_MXFP4_Q4 = 4 };

// A decode step's newest block pooled in the indexer launch (csa_pool_index_topk): one
// block of m raw tokens per sequence, pooled with the same gates into row `row` of the K|V
// cache (bf16 or FP8 K|V rows) and of the MXFP4 indexer-key cache the call then scores.
struct IndexPool {
  bool on = false;
  const void* x = nullptr;       // raw K|V rows of the block (bf16), x_bs rows between sequences
  const void* x2 = nullptr;      // raw indexer-key rows (bf16, DI channels), x2_bs rows apart
  const float* gate = nullptr;   // [B, m]
  const float* bias = nullptr;   // [m]
  int64_t x_bs = 0, x2_bs = 0, C = 0;
  void* y = nullptr;             // K|V cache row `row` of sequence 0, y_bs rows between sequences
  uint8_t* y_scale = nullptr;
  int y_dt = 1;                  // 1 bf16, 4 FP8 K|V rows
  int64_t y_bs = 0;
  int64_t row = 0;
};

struct IndexArgs {
  IndexPool pool;
  const void* qi;
  const uint8_t* qi_scale;   // MXFP4 queries: E8M0 scales [B, Q, HI, DI/32]
  const float* wi;
  const void* ki;
  const uint8_t* ki_scale;
  int kind;
  const int32_t* q_pos;
  int64_t B, Q;
  int HI, DI;
  int64_t N, k_bs;
  int m, k;
  int32_t* out_idx;
  float* out_score;
};

// Workspace bytes of a call (the layout depends on the selection path the call takes).
size_t topk_workspace_bytes(const IndexArgs& a);
hipError_t launch_index_topk(const IndexArgs& a, void* workspace, hipStream_t st);

// ---------------------------------------------------------------- attention
constexpr int kFp8RopeDims = 64;   // bf16 tail of an FP8 K row
// An HCA decode step's newest block pooled inside the attention launch (hca_pool_attend):
// extra workgroups pool each sequence's block of m raw K|V rows into cache entry `row`, the
// last visible entry; the last of them for a sequence adds that entry's contribution (its
// score and its V row) as one more part of the split merge, and the key-range splits stop
// before the entry (the call's N is then the cache's N - 1).
struct AttendPool {
  bool on = false;
  const void* x = nullptr;       // raw K|V rows of the block (bf16, 2D channels), x_bs rows apart
  const float* gate = nullptr;   // [B, m]
  const float* bias = nullptr;   // [m]
  int64_t x_bs = 0;
  int64_t row = 0;
};

struct AttendArgs {
  AttendPool pool;
  const void* q;
  const void* kc;
  const void* vc;
  bool f32;
  bool csa;             // CSA (listed entries) or HCA (every visible entry)
  const int32_t* idx;   // CSA: [B,Q,k]
  int k;
  int m;                // HCA compression ratio
  const void* kw;
  const void* vw;
  const int32_t* win_pos0;
  int64_t L;
  int W;
  const int32_t* q_pos;
  int64_t B, Q;
  int H, D;
  int64_t N, kv_bs;       // kv_bs: rows between batches of kc/vc
  int64_t kv_rs, w_rs;     // elements between rows of kc/vc and of kw/vw (fp8 rows: bytes, K rows)
  float scale;
  // FP8 K/V rows: K = (D - kFp8RopeDims) e4m3 codes then kFp8RopeDims bf16 values, V = D
  // e4m3 codes; decoded value = code * k_scale (K codes) or code * v_scale (V codes).
  bool f8 = false;
  int64_t v_rs = 0, wv_rs = 0;   // bytes between V rows of vc and of vw
  float k_scale = 1.f, v_scale = 1.f;
  void* out;
  float* lse;
};
struct AttendPlan {
  int splits;           // key-range splits per (b, q)
  int chunk;            // keys per split (multiple of the key tile)
  size_t ws_bytes;
  bool supported = true;   // false: the key list is too long for the split limits
};
AttendPlan plan_attend(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p, void* ws, hipStream_t st);

// Debug builds: the flags each source file's kernels recorded since the last read
// (cleared by the read); release builds return 0.
uint32_t debug_flags_attend();
uint32_t debug_flags_index();
uint32_t debug_flags_compress();

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, int64_t R, int D,
                            void* out, bool out_f32, float* lse_out, hipStream_t st);

}  // namespace dsv4
