/*
 * dsv4attn — CSA / HCA long-context attention for MI355X (gfx950), C ABI.
 *
 * The operations follow the method described on:
 *   [CSA] honbul.tistory.com/221, section "CSA: 압축한 뒤, 필요한 기억만 골라서 보기"
 *         (bundle several tokens into one compressed KV entry, let a small indexer
 *         pick the relevant entries for the current token, attend only to those,
 *         and keep recent tokens in a separate sliding window used together with
 *         the compressed memory);
 *   [HCA] same page, section "HCA: 더 강하게 압축하고, 압축된 전체를 보기"
 *         (stronger compression, no sparse selection, attention over every
 *         compressed entry);
 *   [KVC] same page, section "KV cache를 줄이는 방식: 저장 구조까지 바꾼다"
 *         (compressed-entry cache, sliding-window cache and not-yet-compressed tail
 *         kept separately);
 *   [P2]  pogovet.com "DeepSeek-V4: a million-token context that agents can actually
 *         use", 상세 정리 §4 (4x compression by softmax-gated pooling with a learned
 *         positional bias, FP4 lightning indexer choosing top-k compressed blocks per
 *         query, sliding-window branch, 128x compression attended densely) and §5
 *         (KV mostly FP8 with RoPE dims in BF16, indexer in FP4).
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers, row-major, last dimension contiguous.
 *     q_pos and win_pos0 are device arrays too (so calls can be captured in a graph).
 *   - Every call is asynchronous on `stream`; the library never synchronises,
 *     allocates or frees.  Scratch memory comes from the caller's `workspace`.
 *   - Workspace protocol: with workspace == NULL and ws_bytes != NULL the call only
 *     writes the required byte count to *ws_bytes and launches nothing; with a
 *     workspace of at least that size and *ws_bytes set to its size the call runs.
 *     A call whose required size is 0 runs with workspace == NULL and ws_bytes == NULL.
 *     A workspace may be reused by later calls on the same stream; calls that share
 *     one workspace must not run concurrently.
 *   - The caller owns every buffer.  Inputs are read-only; outputs are fully
 *     overwritten; inputs, outputs and workspace must not overlap.
 *   - Size, count and stride arguments must lie in [0, 2^40] (products of two of them
 *     that the calls bound, such as B*Q, are checked without overflow).
 *   - All arguments are validated on the host before anything is launched; a bad
 *     argument returns DSV4_ERR_INVALID_ARG, an unsupported combination
 *     DSV4_ERR_UNSUPPORTED, a too-small workspace DSV4_ERR_WORKSPACE, a failed launch
 *     DSV4_ERR_LAUNCH.  dsv4_last_error() then holds a message (per thread).
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Softmax: lse is the natural-log log-sum-exp of scale * q.k and includes
 *     `scale`.  An empty key set gives o = 0 and lse = -inf.
 *   - MXFP4: two E2M1 codes per byte, the even element in the low nibble; one E8M0
 *     scale byte (exponent + 127) per 32 consecutive elements, in a separate array.
 *     fp8 is OCP E4M3 (bias 7, largest finite 448).  bf16 is IEEE binary32's top half.
 */
#ifndef DSV4ATTN_H
#define DSV4ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSV4_OK = 0,
  DSV4_ERR_INVALID_ARG = 1,
  DSV4_ERR_UNSUPPORTED = 2,
  DSV4_ERR_WORKSPACE = 3,
  DSV4_ERR_LAUNCH = 4
} dsv4_status;

typedef enum {
  DSV4_F32 = 0,
  DSV4_BF16 = 1,
  DSV4_FP8_E4M3 = 2,
  DSV4_MXFP4 = 3,
  DSV4_FP8_KV = 4   /* pooling output only: FP8 K|V rows as read by csa_attend_fp8kv */
} dsv4_dtype;

/* Library version (major * 10000 + minor * 100 + patch). */
int dsv4_version(void);
/* Static name of a status code. */
const char* dsv4_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* dsv4_last_error(void);

/*
 * Instrumentation: arm two events that the NEXT library call made on this thread records
 * immediately before and after its main kernel (the indexer kernel of csa_index_topk, the
 * attention kernel of csa_attend / hca_attend, the pooling kernel of csa_compress, the
 * merge kernel of lse_merge), on that call's stream.  Helper kernels of the same call are
 * outside the pair.  Passing two NULLs disarms.  The events are owned by the caller and
 * must have been created for the device of the call's stream.
 */
dsv4_status dsv4_time_next_kernel(hipEvent_t start, hipEvent_t stop);

/*
 * Debug builds (libdsv4attn_debug.so, compiled with -DDSV4_DEBUG): the kernels also check
 * facts that the release build only enforces by clamping, and record each failed check as
 * a bit (results are the release build's):
 *   1   a top-k scan range's candidate count read back above the keys the range holds
 *   2   the threshold bin, or the count of keys above it, out of range
 *   4   a selected candidate's key index at or past the visible keys
 *   8   a chunk's kept or visible count read back above what the chunk can hold
 *   16  more keys at or above a chunk's kept bin than the chunk keeps
 *   32  an index entry of csa_attend outside [0, N) other than -1 (skipped, as documented)
 *   64  a negative query position (its key set is empty)
 * *flags receives the bits recorded on the current device since the last call, which
 * clears them (0xffffffff if they could not be read).  The call synchronises the device.
 * Release builds set *flags = 0 and return DSV4_ERR_UNSUPPORTED.
 */
dsv4_status dsv4_debug_flags(uint32_t* flags);

/*
 * csa_compress — softmax-gated pooling of disjoint blocks of m raw tokens  [CSA], [HCA], [P2 §4].
 *
 *   y[b,i,:] = sum_{j<m} a_j * x[b, i*m + j, :],
 *   a = softmax_j( gate[b, i*m + j] + pos_bias[j] )          (one gate logit per raw
 *   token, one learned bias per slot; m = 4 for CSA, 128 for HCA; m = 1 is a plain
 *   format conversion, e.g. to quantise indexer keys to MXFP4).
 *
 *   x        [B, x_bstride rows, C] of x_dt (F32 | BF16); batch b starts at row b*x_bstride.
 *            Rows 0..T-1 of each batch are pooled.  x_bstride == 0 means T.
 *   gate     [B, T] f32;  pos_bias [m] f32.
 *   y        [B, y_bstride rows, C] of y_dt (F32 | BF16 | FP8_E4M3), or for MXFP4
 *            [B, y_bstride rows, C/2] bytes plus y_scale [B, y_bstride rows, C/32].
 *            Rows 0..T/m-1 are written.  y_bstride == 0 means T/m.
 *   y_dt = FP8_KV ([P2 §5]: K/V stored mostly in FP8, RoPE dims in BF16): the C channels are
 *            K then V (D = C/2 each, e.g. a [.., 2D] K|V window); each pooled row is written
 *            as one row of C + 64 bytes: K's first D - 64 channels as E4M3 codes, K's last 64
 *            channels as bf16, V's D channels as E4M3 codes (the layout csa_attend_fp8kv
 *            reads with kv_rstride = C + 64 and vc = kc + D + 64).  Codes are
 *            e4m3(y * 2^-e): e = y_scale[0] - 127 for K and y_scale[1] - 127 for V when
 *            y_scale (two device bytes, E8M0) is given, else 0; then k_scale = 2^e_K and
 *            v_scale = 2^e_V for the attention call.  Requires C % 16 == 0, C/2 > 64.
 *   Requires T % m == 0, 1 <= m <= 1024, C % 8 == 0, C <= 1024 (F32 x) or 2048 (BF16 x),
 *   C % 32 == 0 for MXFP4.
 *   Arithmetic: softmax and sums in fp32; rounding to y_dt is nearest-even (fp8 and
 *   MXFP4 saturate; MXFP4 scale = floor(log2 max|y|) - 2 per 32 channels, 0 for an
 *   all-zero group).
 */
dsv4_status csa_compress(const void* x, int x_dt, const float* gate, const float* pos_bias,
                         int64_t B, int64_t T, int64_t C, int32_t m, int64_t x_bstride,
                         void* y, uint8_t* y_scale, int y_dt, int64_t y_bstride,
                         hipStream_t stream);

/*
 * csa_compress2 — csa_compress of two tensors over the same raw blocks in one launch  [CSA],
 * [P2 §4] (a CSA layer pools its K, V and its indexer key with the same gate weights).
 *
 *   y  = csa_compress(x,  gate, pos_bias, m)   with x  [B, x_bstride rows, C],  y  of y_dt
 *   y2 = csa_compress(x2, gate, pos_bias, m)   with x2 [B, x2_bstride rows, C2], y2 of y2_dt
 *   B, T, m, gate and pos_bias are shared; each output is laid out, rounded or quantised
 *   exactly as csa_compress writes it (the same kernel body computes both).
 *   Supported: x_dt = BF16, y_dt in {BF16, FP8_KV}, y2_dt = MXFP4 (y2_scale required);
 *   other combinations return DSV4_ERR_UNSUPPORTED.  Per-tensor constraints and errors as
 *   for csa_compress.  No workspace.
 */
dsv4_status csa_compress2(const void* x, const void* x2, int x_dt, const float* gate, const float* pos_bias,
                          int64_t B, int64_t T, int32_t m, int64_t C, int64_t x_bstride, void* y, uint8_t* y_scale,
                          int y_dt, int64_t y_bstride, int64_t C2, int64_t x2_bstride, void* y2, uint8_t* y2_scale,
                          int y2_dt, int64_t y2_bstride, hipStream_t stream);

/*
 * kv_cache_append — one decode step of cache maintenance around the path  [KVC], [CSA],
 * [HCA], [P2 §4] (a window of recent raw tokens next to the compressed entries).
 *
 * For every sequence b, the new token at position pos[b] is written into a ring window
 * of raw rows, and when it completes a block ((pos[b] + 1) % m == 0) the block's m raw
 * rows are pooled exactly as csa_compress pools them (softmax of gate + pos_bias,
 * weighted sum, rounding or quantisation to y_dt) into compressed row (pos[b] + 1)/m - 1.
 *
 *   x_new     [B, C] of x_dt (F32 | BF16): the new token's raw row (for instance K and V
 *             side by side, C = 2 D, or the raw indexer key).  gate_new [B] f32.
 *   pos       [B] int32 (device): absolute position of the new token of each sequence.
 *   win       [B, L, C] of x_dt, win_gate [B, L] f32: ring window, position p in row
 *             p mod L.  The rows of the block being completed must be present (the
 *             caller appended its earlier tokens).  csa_attend / hca_attend read this
 *             window with win_pos0 == NULL (kw / vw views with w_rstride = C).
 *   L         ring rows: a multiple of m, and at least the attention window W.
 *   pos_bias  [m] f32.
 *   y, y_scale, y_dt, N, y_bstride: the compressed cache, laid out as csa_compress's y
 *             (N rows per sequence, batch stride y_bstride rows, 0 meaning N).  A block
 *             whose row would be >= N, and a sequence with pos[b] < 0, are skipped.
 *   Constraints on C, x_dt and y_dt as for csa_compress.  The window row and the cache
 *   row are overwritten; inputs must not alias them.
 *   Errors: invalid sizes or pointers -> DSV4_ERR_INVALID_ARG; unsupported types ->
 *   DSV4_ERR_UNSUPPORTED; a failed launch -> DSV4_ERR_LAUNCH.  No workspace.
 */
dsv4_status kv_cache_append(const void* x_new, int x_dt, const float* gate_new, const int32_t* pos,
                            int64_t B, int64_t C, void* win, float* win_gate, int64_t L,
                            const float* pos_bias, int32_t m, void* y, uint8_t* y_scale, int y_dt,
                            int64_t N, int64_t y_bstride, hipStream_t stream);

/*
 * csa_index_topk — lightning-indexer scores and per-query top-k block selection  [CSA], [P2 §4].
 *
 *   n(p)      = min(N, floor((p + 1) / m))        blocks complete at or before position p
 *   s[b,q,j]  = sum_{h<HI} wi[b,q,h] * max(0, qi[b,q,h,:] . ki[b,j,:])   for j < n(q_pos[b,q])
 *   out_idx[b,q,:] = the min(k, n) indices with the largest s (equal scores: lower index
 *   first), in ascending order, then -1 padding up to k.
 *
 *   qi        [B, Q, HI, DI] of qi_dt;  wi [B, Q, HI] f32;  q_pos [B, Q] int32 (device).
 *   ki        [B, ki_bstride rows, DI] of ki_dt, or MXFP4 bytes [B, ki_bstride, DI/2] plus
 *             ki_scale [B, ki_bstride, DI/32]; ki_bstride == 0 means N.
 *   (qi_dt, ki_dt) in {(F32,F32), (BF16,BF16), (BF16,MXFP4), (FP8_E4M3,FP8_E4M3),
 *   (MXFP4,MXFP4)}; HI in {4,8,16} and DI in {32,64,128,256} (F32 pair: 1 <= HI <= 16,
 *   1 <= DI <= 256; MXFP4 queries: DI in {128,256}).
 *   MXFP4 queries ([P2 §5]: an FP4 indexer): qi holds the codes [B, Q, HI, DI/2] followed,
 *   in the same allocation, by the E8M0 scales [B, Q, HI, DI/32] (csa_compress with m = 1
 *   writes this layout given y = qi and y_scale = qi + B*Q*HI*DI/2); the products run on
 *   the scaled FP4 MFMA, exact in fp32 for scales within the fp32 range.
 *   1 <= k <= 4096; N < 2^31; B*Q <= 65535.
 *   out_idx   [B, Q, k] int32.   out_score [B, Q, k] f32 (score of each selected index,
 *             -inf on padding) or NULL.
 *   Scores are accumulated in fp32 (bf16 / fp8 / MXFP4 inputs are exact in bf16 / fp8
 *   arithmetic); selection is exact on the fp32 scores.
 */
dsv4_status csa_index_topk(const void* qi, int qi_dt, const float* wi,
                           const void* ki, const uint8_t* ki_scale, int ki_dt,
                           const int32_t* q_pos, int64_t B, int64_t Q, int32_t HI, int32_t DI,
                           int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                           int32_t* out_idx, float* out_score,
                           void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * csa_pool_index_topk — a CSA decode step's pooling and selection in one launch  [CSA],
 * [P2 §4] (the newest block of m raw tokens becomes a compressed entry of both the K|V
 * cache and the indexer-key cache, then every visible entry is scored and the top-k kept).
 *
 *   The result equals  csa_compress2(pool->x, pool->x2, DSV4_BF16, pool->gate,
 *   pool->pos_bias, B, m, m, pool->C, pool->x_bstride, pool->y, pool->y_scale, pool->y_dt,
 *   pool->y_bstride, DI, pool->x2_bstride, ki at row pool->row, ki_scale at row pool->row,
 *   DSV4_MXFP4, ki_bstride or N)  followed by  csa_index_topk(qi, ..., ki, ki_scale, ...)
 *   with the remaining arguments, bit for bit: one block per sequence, pooled with the same
 *   gates into row pool->row (< N) of both caches.  The K|V rows are pooled by extra
 *   workgroups of the indexer launch and the indexer key by the wave that scores it.
 *
 *   pool->x   bf16 raw K|V rows [B, x_bstride rows, C], the block's m rows first (x_bstride
 *             0 means m); pool->x2 the raw indexer-key rows [B, x2_bstride rows, DI].
 *   pool->gate [B, m] f32, pool->pos_bias [m] f32.
 *   pool->y   K|V cache row pool->row of sequence 0 (bf16 [.., C] or FP8 K|V rows of
 *             C + 64 bytes with pool->y_scale as for csa_compress), pool->y_bstride rows
 *             between sequences (0 means N).
 *   ki, ki_scale: MXFP4 indexer keys as for csa_index_topk; row pool->row is written.
 *   qi_dt BF16 or MXFP4; ki_dt MXFP4; m a power of two with m * DI <= 512 (m = 4 with
 *   DI = 128; other m: DSV4_ERR_UNSUPPORTED).  Every other argument, the workspace protocol
 *   and the errors are those of csa_index_topk.
 */
typedef struct dsv4_block_pool {
  const void* x;
  const void* x2;
  const float* gate;
  const float* pos_bias;
  int64_t C;
  int64_t x_bstride, x2_bstride;
  void* y;
  uint8_t* y_scale;
  int y_dt;
  int64_t y_bstride;
  int64_t row;
} dsv4_block_pool;

dsv4_status csa_pool_index_topk(const dsv4_block_pool* pool, const void* qi, int qi_dt, const float* wi, void* ki,
                                uint8_t* ki_scale, int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q,
                                int32_t HI, int32_t DI, int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                                int32_t* out_idx, float* out_score, void* workspace, size_t* ws_bytes,
                                hipStream_t stream);

/*
 * csa_index_topk_noalloc — csa_index_topk for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors are those of csa_index_topk, without
 * the workspace pair.  The call allocates nothing: its scratch is a 48 MiB array owned by
 * the library, one per device, held until the process ends and shared by every call on
 * that device.  A call whose scratch need (the size csa_index_topk's workspace query
 * reports) exceeds 48 MiB returns DSV4_ERR_UNSUPPORTED before any launch (the 1M-context
 * decode, B = 8, N = 262,144, needs about 9 MiB).  Calls that overlap in time on one
 * device race on the array: issue them on one stream, or order them.
 */
dsv4_status csa_index_topk_noalloc(const void* qi, int qi_dt, const float* wi, const void* ki,
                                   const uint8_t* ki_scale, int ki_dt, const int32_t* q_pos, int64_t B, int64_t Q,
                                   int32_t HI, int32_t DI, int64_t N, int64_t ki_bstride, int32_t m, int32_t k,
                                   int32_t* out_idx, float* out_score, hipStream_t stream);

/*
 * csa_attend — attention over the selected compressed entries plus the sliding
 * window, as ONE softmax over the union  [CSA], [P2 §4].
 *
 *   S(b,q) = { kc/vc rows idx[b,q,t] : 0 <= idx < N }  U
 *            { kw/vw rows r < L : q_pos - W < win_pos0[b] + r <= q_pos }
 *   o[b,q,h,:] = sum_{s in S} softmax_s(scale * q[b,q,h,:] . K_s) V_s
 *   lse[b,q,h] = log sum_{s in S} exp(scale * q[b,q,h,:] . K_s)
 *   (multi-query: the H heads share one K/V; a recent token may contribute both through
 *   its compressed entry and through its window row.)
 *
 *   q    [B, Q, H, D];  kc, vc [B, kv_bstride rows, D] (kv_bstride == 0 means N) with
 *        kv_rstride elements from one row to the next (0 means D);
 *   idx  [B, Q, k] int32 (entries outside [0, N) are skipped);
 *   kw, vw [B, L, D]: row r holds position win_pos0[b] + r, w_rstride elements from one row
 *        to the next (0 means D);  win_pos0 [B], q_pos [B, Q].
 *        win_pos0 == NULL selects a ring window: position p lives in row p mod L (the
 *        layout kv_cache_append maintains), every position in (q_pos - W, q_pos] with
 *        p >= 0 is taken to be present, and W <= L is required.
 *   Row strides larger than D let K and V live side by side in one [.., 2D] buffer (then
 *   one csa_compress call pools both).  BF16: strides multiples of 8 elements, rows and
 *   pointers 16-byte aligned.
 *   dt = F32 or BF16 for q, kc, vc, kw, vw and out.  BF16: D in {128, 256, 512} and
 *   H in {16, 32, 48, 64}; F32: D <= 512.  B*Q <= 65535.  out [B, Q, H, D] of dt;  lse [B, Q, H] f32 or NULL.
 *   fp32 accumulation; partial results are merged by log-sum-exp in fp32.
 */
dsv4_status csa_attend(const void* q, const void* kc, const void* vc, int dt,
                       const int32_t* idx, int32_t k,
                       const void* kw, const void* vw, const int32_t* win_pos0, int64_t L, int32_t W,
                       const int32_t* q_pos, int64_t B, int64_t Q, int32_t H, int32_t D,
                       int64_t N, int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float scale,
                       void* out, float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * hca_attend — dense attention over every visible compressed entry plus the sliding
 * window, as ONE softmax  [HCA], [P2 §4].
 *
 *   S(b,q) = { kc/vc rows j < min(N, floor((q_pos + 1) / m)) }  U  window rows as in
 *   csa_attend.  Arguments and layouts as csa_attend, without idx/k and with the
 *   compression ratio m.
 */
dsv4_status hca_attend(const void* q, const void* kc, const void* vc, int dt, int32_t m,
                       const void* kw, const void* vw, const int32_t* win_pos0, int64_t L, int32_t W,
                       const int32_t* q_pos, int64_t B, int64_t Q, int32_t H, int32_t D,
                       int64_t N, int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float scale,
                       void* out, float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * hca_pool_attend — an HCA decode step's pooling and attention in one launch  [HCA],
 * [P2 §4] (the newest block of m raw tokens becomes the last compressed entry, then every
 * visible entry and the window are attended).
 *
 *   The result equals  csa_compress(x, DSV4_BF16, gate, pos_bias, B, m, 2D, m, x_bstride,
 *   kc row N - 1, NULL, DSV4_BF16, kv_bstride or N)  followed by  hca_attend(...) with the
 *   remaining arguments, up to rounding order: the pooled entry (written to row N - 1 of
 *   the K|V cache) enters the softmax as a part of its own, merged by log-sum-exp with the
 *   key ranges over entries [0, N - 1) and the window.  The pooling runs on workgroups of
 *   the attention launch that the key ranges leave free.
 *
 *   x         bf16 raw K|V rows [B, x_bstride rows, 2D], the block's m rows first (K then V
 *             channels, as the cache rows; x_bstride 0 means m);  gate [B, m], pos_bias [m].
 *   kc, vc    one buffer of K|V rows: vc = kc + D elements, kv_rstride >= 2D.
 *   dt = DSV4_BF16, D = 512, Q < 16, N >= 1.  Every other argument, the workspace protocol
 *   and the errors are those of hca_attend (the workspace also holds the pooled entry's
 *   per-query scores).  Row N - 1 is written by this call and read back by the merge
 *   launch that ends it; the attention workgroups never read it, so no ordering between
 *   workgroups of one launch is needed.  x may be the window's rows (both are only read),
 *   but not row N - 1 of the cache.
 */
dsv4_status hca_pool_attend(const void* x, const float* gate, const float* pos_bias, int64_t x_bstride,
                            const void* q, const void* kc, const void* vc, int dt, int32_t m, const void* kw,
                            const void* vw, const int32_t* win_pos0, int64_t L, int32_t W, const int32_t* q_pos,
                            int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int64_t kv_bstride,
                            int64_t kv_rstride, int64_t w_rstride, float scale, void* out, float* lse, void* workspace,
                            size_t* ws_bytes, hipStream_t stream);

/*
 * csa_attend_fp8kv, hca_attend_fp8kv — csa_attend / hca_attend over K/V caches stored in
 * FP8 with the RoPE dims of K kept in BF16  [P2 §5] (most of each KV entry in FP8, the
 * RoPE dims in BF16), dequantised inside the attention kernel.
 *
 *   K row (kc and kw): D - d_rope E4M3 codes (bytes), then d_rope bf16 values (the RoPE
 *       dims, the last d_rope dims of the head), i.e. D + d_rope bytes.
 *   V row (vc and vw): D E4M3 codes.
 *   Decoded K = [k_scale * e4m3(code) for the code dims, the bf16 values as they are];
 *   decoded V = v_scale * e4m3(code).  One scale per tensor kind (compressed and window
 *   rows share it).  The result is the bf16 call's result on the decoded K and V: the
 *   codes are decoded exactly, k_scale multiplies the fp32 partial scores of the code
 *   dims and v_scale the fp32 output, so both are applied without an extra rounding.
 *   q, out: bf16 as in csa_attend; lse f32.  D = 512, d_rope = 64, H in {16, 32, 48, 64}.
 *   kv_rstride, w_rstride: BYTES from one row to the next, shared by K and V rows (so a K
 *   row and its V row may sit side by side in one row of D + d_rope + D bytes); 0 means
 *   D + d_rope for K rows and D for V rows.  Nonzero strides: multiples of 16, >= D +
 *   d_rope.  kc, vc, kw, vw 16-byte aligned.  k_scale, v_scale finite.
 *   Every other argument, the workspace protocol and the errors are as for csa_attend /
 *   hca_attend.
 */
dsv4_status csa_attend_fp8kv(const void* q, const void* kc, const void* vc, const int32_t* idx, int32_t k,
                             const void* kw, const void* vw, const int32_t* win_pos0, int64_t L, int32_t W,
                             const int32_t* q_pos, int64_t B, int64_t Q, int32_t H, int32_t D, int32_t d_rope,
                             int64_t N, int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float k_scale,
                             float v_scale, float scale, void* out, float* lse, void* workspace, size_t* ws_bytes,
                             hipStream_t stream);
dsv4_status hca_attend_fp8kv(const void* q, const void* kc, const void* vc, int32_t m, const void* kw,
                             const void* vw, const int32_t* win_pos0, int64_t L, int32_t W, const int32_t* q_pos,
                             int64_t B, int64_t Q, int32_t H, int32_t D, int32_t d_rope, int64_t N,
                             int64_t kv_bstride, int64_t kv_rstride, int64_t w_rstride, float k_scale,
                             float v_scale, float scale, void* out, float* lse, void* workspace, size_t* ws_bytes,
                             hipStream_t stream);

/*
 * lse_merge — combine attention results over P disjoint key sets (e.g. the compressed
 * part and the window part, or the shards of a split key range) into the result over
 * their union.  Source: the pages describe no merge step; they only say that the
 * compressed memory and the recent raw window are used together ([CSA], [P2 §4]).  The
 * merge comes from the workload definition instead (the 1M-context HCA decode combines
 * its compressed branch and its window branch with it), and it is exact: one softmax over
 * the union of the key sets equals the log-sum-exp merge of the softmaxes over its parts.
 *
 *   M = max_p lse_p;  lse = M + log sum_p exp(lse_p - M);  o = sum_p exp(lse_p - lse) o_p
 *   (a part with lse = -inf is empty; all parts empty -> o = 0, lse = -inf).
 *
 *   o_parts [P, R, D] f32;  lse_parts [P, R] f32;  out [R, D] of out_dt (F32 | BF16);
 *   lse_out [R] f32 or NULL.  1 <= P <= 1024; D % 4 == 0, D <= 4096.
 */
dsv4_status lse_merge(const float* o_parts, const float* lse_parts, int32_t P, int64_t R, int32_t D,
                      void* out, int out_dt, float* lse_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSV4ATTN_H */
