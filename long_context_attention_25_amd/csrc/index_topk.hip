// Lightning-indexer scoring and per-query top-k block selection for gfx950.
//
// A small indexer scores every visible compressed block for the current query and
// only the best k blocks go on to attention (honbul.tistory.com/221, "CSA: 압축한
// 뒤, 필요한 기억만 골라서 보기"; pogovet.com 상세 정리 §4 and §5: an FP4 lightning
// indexer picks the top-k compressed blocks per query).  Score of block j:
//     s_j = sum_h w_h * max(0, q_h . k_j)            (j < floor((p+1)/m) only)
//
// Decode path (few query rows, very long rows):
//   1. index kernel: streams the keys once (bf16, fp8 e4m3 or MXFP4 decoded to bf16
//      in registers) and computes the [heads x keys] dot products with MFMA
//      (16 rows = QPT queries x HI heads, 16 keys per tile, K = 32 per step).  The
//      epilogue applies ReLU, the head weights and the head sum, writes the fp32
//      scores and adds the top 12 bits of each score's order-preserving key into a
//      per-row histogram (LDS histogram, then one global atomic per non-empty bin).
//   2. select kernel: every workgroup finds the threshold bin of its row from the
//      histogram, writes the bitmap words of its key range for the keys strictly
//      above the bin, and appends the keys inside the bin as candidates.  The last
//      workgroup of a row (atomic counter) radix-selects the remaining candidates by
//      (score, lower index first), sets their bits, and compacts the bitmap into
//      ascending indices.
// The result is exact on the fp32 scores and independent of scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace dsv4 {

namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerIter = 256;   // 4 waves x 4 tiles x 16 keys
constexpr int kMaxSelGroups = 64;   // select workgroups per row at most
constexpr int kSelCounters = 1 + kMaxSelGroups;
constexpr int kCandCap = 4096;      // candidates staged in LDS by the finishing workgroup

__device__ __forceinline__ uint32_t vis_blocks(const int32_t* q_pos, int64_t row, int m, int64_t N) {
  int64_t p = q_pos[row];
  int64_t n = (p + 1) / m;
  if (p < 0) n = 0;
  return (uint32_t)(n < N ? n : N);
}

// Block-wide exclusive prefix sum of one value per thread (256 threads); returns the
// exclusive prefix and writes the total to *total.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds4, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) lds4[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = lds4[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ void clear_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// Writes one score and counts it in the LDS histogram of its query slot.
__device__ __forceinline__ void emit_score(float* scores, uint32_t* hist_l, int64_t row, int64_t sstride,
                                           int64_t N, int64_t key, uint32_t nvis, float v) {
  if (key >= N) return;
  bool vis = key < (int64_t)nvis;
  scores[row * sstride + key] = vis ? v : -INFINITY;
  if (vis) atomicAdd(&hist_l[score_key(v) >> (32 - kHistBits)], 1u);
}

__device__ __forceinline__ void flush_hist(const uint32_t* hist_l, uint32_t* hist_g, int64_t row) {
  for (int bin = threadIdx.x; bin < kHistBins; bin += kThreads) {
    uint32_t c = hist_l[bin];
    if (c) atomicAdd(&hist_g[row * kHistBins + bin], c);
  }
}

// ------------------------------------------------------------------ fp32 keys (VALU)
__global__ __launch_bounds__(kThreads) void index_f32_kernel(
    const float* __restrict__ qi, const float* __restrict__ wi, const float* __restrict__ ki,
    const int32_t* __restrict__ q_pos, int64_t N, int64_t k_bs, int64_t Q, int HI, int DI, int m,
    float* __restrict__ scores, int64_t sstride, uint32_t* __restrict__ hist_g) {
  extern __shared__ uint32_t sm[];
  uint32_t* hist_l = sm;
  float* qs = reinterpret_cast<float*>(sm + kHistBins);
  float* ws = qs + HI * DI;
  const int64_t row = blockIdx.y;            // b * Q + q
  const int64_t b = row / Q;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist_l[i] = 0u;
  for (int i = threadIdx.x; i < HI * DI; i += kThreads) qs[i] = qi[row * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kThreads) ws[i] = wi[row * HI + i];
  __syncthreads();
  const uint32_t nvis = vis_blocks(q_pos, row, m, N);
  int64_t key = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (key < N) {
    float s = 0.f;
    if (key < (int64_t)nvis) {
      const float* kr = ki + (b * k_bs + key) * DI;
      for (int h = 0; h < HI; ++h) {
        float d = 0.f;
        for (int t = 0; t < DI; ++t) d = fmaf(qs[h * DI + t], kr[t], d);
        s = fmaf(ws[h], fmaxf(d, 0.f), s);
      }
    }
    emit_score(scores, hist_l, row, sstride, N, key, nvis, s);
  }
  __syncthreads();
  flush_hist(hist_l, hist_g, row);
}

// ------------------------------------------------------------------ MFMA key streams
// Per lane: key (lane % 16) of a 16-key tile and the contiguous quarter g = lane / 16
// of its DI dims; k-step c of the MFMA takes dims g*DI/4 + 8c .. +7 of both the key and
// the query row, which pairs every key element with the same query element.
template <int KIND, int DI>
struct KeyTile;

template <int DI>
struct KeyTile<KEY_BF16, DI> {
  static constexpr int KS = DI / 32;
  uint4 w[KS];
  __device__ void load(const uint8_t* kbase, const uint8_t*, int64_t key, int g, bool ok) {
    const uint4* p = reinterpret_cast<const uint4*>(kbase + key * (DI * 2) + g * (DI / 2));
#pragma unroll
    for (int c = 0; c < KS; ++c) w[c] = ok ? p[c] : make_uint4(0, 0, 0, 0);
  }
  __device__ bf16x8 op(int c) const { return bit_cast_to<bf16x8>(w[c]); }
};

template <int DI>
struct KeyTile<KEY_MXFP4, DI> {
  static constexpr int KS = DI / 32;
  uint32_t w[KS];
  uint32_t sc;   // up to 2 scale bytes for this lane's dims
  __device__ void load(const uint8_t* kbase, const uint8_t* sbase, int64_t key, int g, bool ok) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(kbase + key * (DI / 2) + g * (DI / 8));
#pragma unroll
    for (int c = 0; c < KS; ++c) w[c] = ok ? p[c] : 0u;
    const uint8_t* s = sbase + key * (DI / 32) + (g * (DI / 4)) / 32;
    if constexpr (DI == 256) sc = ok ? (uint32_t)s[0] | ((uint32_t)s[1] << 8) : 0x7f7fu;
    else sc = ok ? (uint32_t)s[0] : 0x7fu;
  }
  __device__ bf16x8 op(int c) const {
    // scale byte of k-step c: dims g*DI/4 + 8c lie in group (g*DI/4 + 8c)/32
    uint32_t e = (DI == 256) ? ((sc >> ((c >= 4) ? 8 : 0)) & 0xffu) : (sc & 0xffu);
    float scale = __uint_as_float(e << 23);      // 2^(e-127); e == 0 maps to 0 (not produced here)
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 0);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 1);
    bf16x2 cc = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 2);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[c], scale, 3);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = cc[0]; r[5] = cc[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
};

template <int DI>
struct KeyTile<KEY_FP8, DI> {
  static constexpr int KS = DI / 32;
  uint2 w[KS];
  __device__ void load(const uint8_t* kbase, const uint8_t*, int64_t key, int g, bool ok) {
    const uint2* p = reinterpret_cast<const uint2*>(kbase + key * DI + g * (DI / 4));
#pragma unroll
    for (int c = 0; c < KS; ++c) w[c] = ok ? p[c] : make_uint2(0, 0);
  }
  __device__ long op(int c) const { return __builtin_bit_cast(long, w[c]); }
};

template <int KIND, int DI, int HI>
__global__ __launch_bounds__(kThreads) void index_mfma_kernel(
    const uint8_t* __restrict__ qi, const float* __restrict__ wi, const uint8_t* __restrict__ ki,
    const uint8_t* __restrict__ ksc, const int32_t* __restrict__ q_pos, int64_t N, int64_t k_bs,
    int64_t Q, int m, int64_t chunk, float* __restrict__ scores, int64_t sstride, uint32_t* __restrict__ hist_g) {
  constexpr int QPT = 16 / HI;          // queries per 16-row MFMA tile
  constexpr int KS = DI / 32;
  constexpr int GPQ = HI / 4;           // lane groups per query slot
  extern __shared__ uint32_t hist_l[];  // [QPT][kHistBins]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t QT = (Q + QPT - 1) / QPT;
  const int64_t b = blockIdx.y / QT, qt = blockIdx.y % QT;
  const int nq = (int)((Q - qt * QPT) < QPT ? (Q - qt * QPT) : QPT);

  for (int i = threadIdx.x; i < nq * kHistBins; i += kThreads) hist_l[i] = 0u;

  // A operand: query rows (row = lane % 16 = qslot * HI + head)
  const int r = col;
  const int qs_a = r / HI, h_a = r % HI;
  const bool qa_ok = qs_a < nq;
  const int64_t qrow_a = (b * Q + qt * QPT + (qa_ok ? qs_a : 0)) * HI + h_a;
  uint4 qa16[KS];   // bf16 queries
  uint2 qa8[KS];    // fp8 queries
  if constexpr (KIND == KEY_FP8) {
    const uint2* p = reinterpret_cast<const uint2*>(qi + qrow_a * DI + g * (DI / 4));
#pragma unroll
    for (int c = 0; c < KS; ++c) qa8[c] = qa_ok ? p[c] : make_uint2(0, 0);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(qi + (qrow_a * DI + g * (DI / 4)) * 2);
#pragma unroll
    for (int c = 0; c < KS; ++c) qa16[c] = qa_ok ? p[c] : make_uint4(0, 0, 0, 0);
  }
  // epilogue weights: accumulator row 4g+i -> (slot (4g+i)/HI, head (4g+i)%HI)
  const int qs_c = (4 * g) / HI;
  const bool qc_ok = qs_c < nq;
  const int64_t row_c = b * Q + qt * QPT + (qc_ok ? qs_c : 0);
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = qc_ok ? wi[row_c * HI + ((4 * g + i) % HI)] : 0.f;
  const uint32_t nvis = qc_ok ? vis_blocks(q_pos, row_c, m, N) : 0u;
  const bool owner = qc_ok && (g % GPQ) == 0;
  __syncthreads();

  const uint8_t* kbase;
  const uint8_t* sbase = nullptr;
  if constexpr (KIND == KEY_BF16) kbase = ki + b * k_bs * DI * 2;
  else if constexpr (KIND == KEY_FP8) kbase = ki + b * k_bs * DI;
  else {
    kbase = ki + b * k_bs * (DI / 2);
    sbase = ksc + b * k_bs * (DI / 32);
  }

  // Each wave takes 64 consecutive keys (4 tiles) per step; the next step's tiles are
  // loaded before this step's are used.  Key indices past the range are clamped to its
  // last key, so loads never branch; only the score write is guarded.
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  int64_t c1 = c0 + chunk;
  if (c1 > N) c1 = N;
  const int64_t klast = c1 - 1;
  KeyTile<KIND, DI> cur[4], nxt[4];
  int64_t base = c0 + wave * 64;
  if (base < c1) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t key = base + u * 16 + col;
      cur[u].load(kbase, sbase, key < klast ? key : klast, g, true);
    }
  }
  for (; base < c1; base += kKeysPerIter) {
    const int64_t nb = base + kKeysPerIter;
    if (nb < c1) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t key = nb + u * 16 + col;
        nxt[u].load(kbase, sbase, key < klast ? key : klast, g, true);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        if constexpr (KIND == KEY_FP8) acc = mfma_fp8(__builtin_bit_cast(long, qa8[c]), cur[u].op(c), acc);
        else acc = mfma_bf16(bit_cast_to<bf16x8>(qa16[c]), cur[u].op(c), acc);
      }
      float v = wv[0] * fmaxf(acc[0], 0.f);
      v = fmaf(wv[1], fmaxf(acc[1], 0.f), v);
      v = fmaf(wv[2], fmaxf(acc[2], 0.f), v);
      v = fmaf(wv[3], fmaxf(acc[3], 0.f), v);
      if constexpr (GPQ >= 2) v += __shfl_xor(v, 16);
      if constexpr (GPQ >= 4) v += __shfl_xor(v, 32);
      const int64_t key = base + u * 16 + col;
      if (owner && key < c1) emit_score(scores, hist_l + qs_c * kHistBins, row_c, sstride, N, key, nvis, v);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
  }
  __syncthreads();
  for (int s = 0; s < nq; ++s) flush_hist(hist_l + s * kHistBins, hist_g, b * Q + qt * QPT + s);
}

// ------------------------------------------------------------------ selection
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist_g, uint32_t* __restrict__ counters,
    uint32_t* __restrict__ bitmap, uint64_t* __restrict__ cand, const int32_t* __restrict__ q_pos,
    int64_t N, int64_t sstride, int64_t words, int m, int k, int64_t chunk, int32_t* __restrict__ out_idx,
    float* __restrict__ out_score) {
  __shared__ uint32_t sh_misc[16];
  __shared__ uint32_t sh_h[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const uint32_t n = vis_blocks(q_pos, row, m, N);
  const uint32_t kk = (uint32_t)k < n ? (uint32_t)k : n;

  // ---- threshold bin: largest t with #(keys with bin >= t) >= kk
  const uint32_t* hr = hist_g + row * kHistBins;
  uint32_t hv[kHistBins / kThreads];
  uint32_t tsum = 0;
#pragma unroll
  for (int i = 0; i < kHistBins / kThreads; ++i) {
    hv[i] = hr[tid * (kHistBins / kThreads) + i];
    tsum += hv[i];
  }
  if (tid == 0) { sh_misc[4] = kHistBins; sh_misc[5] = 0; }
  uint32_t total;
  uint32_t excl = block_excl_scan(tsum, sh_misc, &total);
  uint32_t above = total - excl - tsum;         // keys in higher threads' bins
  if (kk > 0 && above < kk && kk <= above + tsum) {
    uint32_t acc = above;
    for (int i = kHistBins / kThreads - 1; i >= 0; --i) {
      if (acc + hv[i] >= kk) { sh_misc[4] = tid * (kHistBins / kThreads) + i; sh_misc[5] = acc; break; }
      acc += hv[i];
    }
  }
  __syncthreads();
  const uint32_t tbin = sh_misc[4], cnt_above = sh_misc[5];

  // ---- bitmap words of this range (keys strictly above the bin) + candidates (in the bin).
  // Thread t owns 64 consecutive keys per 16384-key group: 16 float4 loads in flight, its
  // two bitmap words built in registers, its candidates placed by a block-wide scan into
  // this workgroup's own slice of the candidate buffer.
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  int64_t c1 = c0 + chunk;
  if (c1 > (int64_t)n) c1 = n;
  uint32_t* bm = bitmap + row * words;
  uint64_t* cr = cand + row * N + c0;
  uint32_t* rc = counters + row * kSelCounters;     // [0] arrivals, [1 + w] candidates of workgroup w
  const float* srow_in = scores + row * sstride;
  uint32_t cand_base = 0;
  for (int64_t gbase = c0; gbase < c1; gbase += (int64_t)kThreads * 64) {
    const int64_t kb = gbase + (int64_t)tid * 64;
    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = kb < c1 ? reinterpret_cast<const float4*>(srow_in + kb)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t wlo = 0, whi = 0, ncand = 0;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const float sv = (e & 3) == 0 ? v[e >> 2].x : (e & 3) == 1 ? v[e >> 2].y : (e & 3) == 2 ? v[e >> 2].z : v[e >> 2].w;
      const uint32_t bin = score_key(sv) >> (32 - kHistBits);
      const bool in = kb + e < c1;
      if (in && bin > tbin) {
        if (e < 32) wlo |= 1u << e;
        else whi |= 1u << (e - 32);
      }
      ncand += (in && bin == tbin) ? 1u : 0u;
    }
    if (kb < c1) *reinterpret_cast<uint2*>(bm + kb / 32) = make_uint2(wlo, whi);
    uint32_t gtot;
    uint32_t pos = cand_base + block_excl_scan(ncand, sh_misc, &gtot);
    if (ncand) {
#pragma unroll
      for (int e = 0; e < 64; ++e) {
        const float sv = (e & 3) == 0 ? v[e >> 2].x : (e & 3) == 1 ? v[e >> 2].y : (e & 3) == 2 ? v[e >> 2].z : v[e >> 2].w;
        const uint32_t key = score_key(sv);
        if (kb + e < c1 && (key >> (32 - kHistBits)) == tbin)
          cr[pos++] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)(kb + e));
      }
    }
    cand_base += gtot;
  }
  if (tid == 0) rc[1 + blockIdx.x] = cand_base;

  // ---- the last workgroup of the row finishes the selection (every thread releases its
  // own bitmap / candidate stores before the arrival is counted)
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t prev = atomicAdd(&rc[0], 1u);
    sh_misc[6] = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!sh_misc[6]) return;
  __threadfence();

  __shared__ uint32_t sh_cnt[kMaxSelGroups];
  for (int w = tid; w < (int)gridDim.x; w += kThreads)
    sh_cnt[w] = __hip_atomic_load(&rc[1 + w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint64_t* call = cand + row * N;
  // Stage the candidates in LDS when they fit (the usual case: about one histogram bin of
  // keys); otherwise the passes below read them from each workgroup's slice in turn.
  __shared__ uint64_t sh_cand[kCandCap];
  __shared__ uint32_t sh_pre[kMaxSelGroups + 1];
  if (tid == 0) {
    uint32_t acc_ = 0;
    for (int w = 0; w < (int)gridDim.x; ++w) {
      sh_pre[w] = acc_;
      acc_ += sh_cnt[w];
    }
    sh_pre[gridDim.x] = acc_;
  }
  __syncthreads();
  const uint32_t c = sh_pre[gridDim.x];
  const bool in_lds = c <= (uint32_t)kCandCap;
  if (in_lds) {
    // kCandCap / kThreads = 16 slots per thread: all loads issued before any is stored
    constexpr int kPer = kCandCap / kThreads;
    uint64_t vals[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t f = tid + u * kThreads;
      int w = 0;
      while (w + 1 < (int)gridDim.x && sh_pre[w + 1] <= f) ++w;
      vals[u] = f < c ? call[(int64_t)w * chunk + (f - sh_pre[w])] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t f = tid + u * kThreads;
      if (f < c) sh_cand[f] = vals[u];
    }
    __syncthreads();
  }
#define DSV4_FOR_CAND(body)                                               \
  if (in_lds) {                                                           \
    for (uint32_t f_ = tid; f_ < c; f_ += kThreads) {                     \
      const uint64_t comp = sh_cand[f_];                                  \
      body                                                                \
    }                                                                     \
  } else {                                                                \
    for (int w_ = 0; w_ < (int)gridDim.x; ++w_) {                         \
      const uint64_t* cw_ = call + (int64_t)w_ * chunk;                   \
      for (uint32_t i_ = tid; i_ < sh_cnt[w_]; i_ += kThreads) {          \
        const uint64_t comp = cw_[i_];                                    \
        body                                                              \
      }                                                                   \
    }                                                                     \
  }
  uint32_t need = kk - cnt_above;
  // threshold on the composite key (score key << 32 | ~index): select comp >= thr
  uint64_t prefix = (uint64_t)tbin << (64 - kHistBits);
  uint64_t thr;
  bool none = (need == 0);
  if (need == c) {
    thr = 0;
  } else {
    int hi = 64 - kHistBits;                    // bits [hi-1 : 0] still open
    while (true) {
      int wd = hi < 8 ? hi : 8;
      int sh = hi - wd;
      sh_h[tid] = 0u;
      __syncthreads();
      DSV4_FOR_CAND(if ((comp >> hi) == (prefix >> hi)) atomicAdd(&sh_h[(comp >> sh) & ((1u << wd) - 1u)], 1u);)
      __syncthreads();
      uint32_t hcount = (tid < (1 << wd)) ? sh_h[tid] : 0u;
      uint32_t tot;
      uint32_t ex = block_excl_scan(hcount, sh_misc, &tot);
      uint32_t gt = tot - ex - hcount;          // candidates with a larger digit
      if (tid < (1 << wd) && gt < need && need <= gt + hcount) {
        sh_misc[8] = tid;
        sh_misc[9] = gt;
        sh_misc[10] = hcount;
      }
      __syncthreads();
      uint32_t d = sh_misc[8];
      need -= sh_misc[9];
      prefix |= (uint64_t)d << sh;
      bool done = (sh_misc[10] == need) || sh == 0;
      __syncthreads();
      hi = sh;
      if (done) break;
    }
    thr = prefix;
  }
  if (!none) {
    DSV4_FOR_CAND(if (comp >= thr) {
      const uint32_t j = ~(uint32_t)comp;
      atomicOr(&bm[j / 32], 1u << (j % 32));
    })
  }
  __threadfence();
  __syncthreads();

  // ---- compact the bitmap into ascending indices: rounds of 32 words (1024 keys) per
  // thread, loaded as 8 x 16 bytes (the fence above made the other workgroups' words and
  // the atomics visible to plain loads)
  const int64_t wn = ((int64_t)n + 31) / 32;
  int32_t* orow = out_idx + row * k;
  float* srow = out_score ? out_score + row * k : nullptr;
  uint32_t base_off = 0;
  for (int64_t r0 = 0; r0 < wn; r0 += 32 * kThreads) {
    const int64_t w0 = r0 + (int64_t)tid * 32;
    uint32_t wv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = (w0 + 4 * i < wn) ? *reinterpret_cast<const uint4*>(bm + w0 + 4 * i) : make_uint4(0, 0, 0, 0);
      wv[4 * i] = v.x; wv[4 * i + 1] = v.y; wv[4 * i + 2] = v.z; wv[4 * i + 3] = v.w;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) cnt += __popc(w0 + i < wn ? wv[i] : 0u);
    uint32_t rtot;
    uint32_t off = base_off + block_excl_scan(cnt, sh_misc, &rtot);
    for (int i = 0; i < 32; ++i) {
      uint32_t bits = w0 + i < wn ? wv[i] : 0u;
      while (bits) {
        int bpos = __ffs(bits) - 1;
        bits &= bits - 1;
        int64_t j = (w0 + i) * 32 + bpos;
        if (off < (uint32_t)k) {
          orow[off] = (int32_t)j;
          if (srow) srow[off] = scores[row * sstride + j];
        }
        ++off;
      }
    }
    base_off += rtot;
  }
  const uint32_t tot = base_off;
  for (int64_t p = (int64_t)tot + tid; p < k; p += kThreads) {
    orow[p] = -1;
    if (srow) srow[p] = -INFINITY;
  }
}

template <int KIND, int DI>
hipError_t launch_mfma_di(const IndexArgs& a, float* scores, uint32_t* hist, int64_t chunk, hipStream_t st) {
  int QPT = 16 / a.HI;
  int64_t QT = (a.Q + QPT - 1) / QPT;
  dim3 grid((unsigned)((a.N + chunk - 1) / chunk), (unsigned)(a.B * QT));
  size_t smem = (size_t)(a.Q < QPT ? a.Q : QPT) * kHistBins * sizeof(uint32_t);
  const uint8_t* qi = reinterpret_cast<const uint8_t*>(a.qi);
  const uint8_t* ki = reinterpret_cast<const uint8_t*>(a.ki);
#define DSV4_IDX_LAUNCH(HIv)                                                                                  \
  DSV4_LAUNCH_MAIN((index_mfma_kernel<KIND, DI, HIv>), grid, dim3(kThreads), smem, st, qi, a.wi, ki,        \
                     a.ki_scale, a.q_pos, a.N, a.k_bs, a.Q, a.m, chunk, scores, ((a.N + 63) / 64) * 64, hist)
  switch (a.HI) {
    case 4: DSV4_IDX_LAUNCH(4); break;
    case 8: DSV4_IDX_LAUNCH(8); break;
    default: DSV4_IDX_LAUNCH(16); break;
  }
#undef DSV4_IDX_LAUNCH
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_mfma(const IndexArgs& a, float* scores, uint32_t* hist, int64_t chunk, hipStream_t st) {
  switch (a.DI) {
    case 32: return launch_mfma_di<KIND, 32>(a, scores, hist, chunk, st);
    case 64: return launch_mfma_di<KIND, 64>(a, scores, hist, chunk, st);
    case 128: return launch_mfma_di<KIND, 128>(a, scores, hist, chunk, st);
    default: return launch_mfma_di<KIND, 256>(a, scores, hist, chunk, st);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t topk_workspace_bytes(int64_t R, int64_t N) {
  int64_t words = ((N + 127) / 128) * 4;   // rows of 16-byte multiples
  const int64_t sstride = ((N + 63) / 64) * 64;
  return align256((size_t)R * sstride * 4) + align256((size_t)R * kHistBins * 4 + (size_t)R * kSelCounters * 4) +
         align256((size_t)R * words * 4) + align256((size_t)R * N * 8);
}

TopkWorkspace topk_workspace_carve(void* base, int64_t R, int64_t N) {
  int64_t words = ((N + 127) / 128) * 4;   // rows of 16-byte multiples
  uint8_t* p = reinterpret_cast<uint8_t*>(base);
  TopkWorkspace w;
  w.scores = reinterpret_cast<float*>(p);
  p += align256((size_t)R * (((N + 63) / 64) * 64) * 4);
  w.hist = reinterpret_cast<uint32_t*>(p);
  w.counters = w.hist + R * kHistBins;
  p += align256((size_t)R * kHistBins * 4 + (size_t)R * kSelCounters * 4);
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * words * 4);
  w.cand = reinterpret_cast<uint64_t*>(p);
  return w;
}

hipError_t launch_index_topk(const IndexArgs& a, const TopkWorkspace& ws, hipStream_t st) {
  const int64_t R = a.B * a.Q;
  if (R == 0) return hipSuccess;
  const int64_t nclear = R * kHistBins + R * kSelCounters;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclear + 1023) / 1024 < 256 ? (nclear + 1023) / 1024 : 256)),
                     dim3(1024), 0, st, ws.hist, nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N > 0) {
    if (a.kind == KEY_F32) {
      dim3 grid((unsigned)((a.N + kThreads - 1) / kThreads), (unsigned)R);
      size_t smem = (kHistBins + (size_t)a.HI * a.DI + a.HI) * 4;
      DSV4_LAUNCH_MAIN(index_f32_kernel, grid, dim3(kThreads), smem, st, reinterpret_cast<const float*>(a.qi),
                         a.wi, reinterpret_cast<const float*>(a.ki), a.q_pos, a.N, a.k_bs, a.Q, a.HI, a.DI, a.m,
                         ws.scores, ((a.N + 63) / 64) * 64, ws.hist);
      e = hipGetLastError();
    } else {
      // about two workgroups per CU over the whole call, each a multiple of 256 keys
      int QPT = 16 / a.HI;
      int64_t rows = a.B * ((a.Q + QPT - 1) / QPT);
      int64_t per = (a.N * rows + 511) / 512;
      int64_t chunk = ((per + kKeysPerIter - 1) / kKeysPerIter) * kKeysPerIter;
      if (chunk < kKeysPerIter) chunk = kKeysPerIter;
      if (a.kind == KEY_BF16) e = launch_mfma<KEY_BF16>(a, ws.scores, ws.hist, chunk, st);
      else if (a.kind == KEY_FP8) e = launch_mfma<KEY_FP8>(a, ws.scores, ws.hist, chunk, st);
      else e = launch_mfma<KEY_MXFP4>(a, ws.scores, ws.hist, chunk, st);
    }
    if (e != hipSuccess) return e;
  }
  // selection: ranges of 16384 keys (more per range past 64 ranges per row)
  const int64_t kGroup = (int64_t)kThreads * 64;
  int64_t schunk = kGroup;
  if ((a.N + schunk - 1) / schunk > kMaxSelGroups)
    schunk = ((a.N + kMaxSelGroups * kGroup - 1) / (kMaxSelGroups * kGroup)) * kGroup;
  int64_t nsel = (a.N + schunk - 1) / schunk;
  if (nsel < 1) nsel = 1;
  int64_t words = ((a.N + 127) / 128) * 4;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)nsel, (unsigned)R), dim3(kThreads), 0, st, ws.scores, ws.hist,
                     ws.counters, ws.bitmap, ws.cand, a.q_pos, a.N, ((a.N + 63) / 64) * 64, words, a.m, a.k, schunk,
                     a.out_idx, a.out_score);
  return hipGetLastError();
}

}  // namespace dsv4
