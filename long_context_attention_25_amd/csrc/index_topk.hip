// Lightning-indexer scoring and per-query top-k block selection for gfx950.
//
// A small indexer scores every visible compressed block for the current query and
// only the best k blocks go on to attention (honbul.tistory.com/221, "CSA: 압축한
// 뒤, 필요한 기억만 골라서 보기"; pogovet.com 상세 정리 §4 and §5: an FP4 lightning
// indexer picks the top-k compressed blocks per query).  Score of block j:
//     s_j = sum_h w_h * max(0, q_h . k_j)            (j < floor((p+1)/m) only)
//
// Index kernel (every call): streams the keys once (bf16, fp8 e4m3 or MXFP4 decoded to
// bf16 in registers) and computes the [heads x keys] dot products with MFMA (16 rows =
// QPT queries x HI heads, 16 keys per tile, K = 32 per step; fp8 keys with DI >= 128 and
// MXFP4 queries: the scaled MFMA, K = 128 per step).  Its epilogue applies ReLU, the head
// weights and the head sum, and counts the top 12 bits of each score's order-preserving
// key in an LDS histogram.
// Decode-shaped calls (one query tile per workgroup, N <= 2^18): two launches.
//   1. the index kernel keeps its chunk's scores in LDS and ends with a local selection:
//      the whole histogram bins holding the chunk's best keys (at most klocal of them)
//      become the chunk's candidates; the scores go to the workspace;
//   2. one workgroup per row selects the top-k among the chunks' candidates, widening the
//      rare chunk that could hide more winners than it kept (select_local_kernel).
// Other calls (many queries per sequence, fp32 keys, longer rows): five launches.
//   0. the row histograms are cleared; 1. the index kernel adds its LDS histogram to them
//   and writes the scores; 2. one workgroup per row finds the row's threshold bin; 3. a
//   chip-wide scan pass (rows x key ranges) marks the keys above it in a bitmap and
//   collects the keys inside it; 4. one workgroup per row radix-selects those candidates
//   and compacts the bitmap.
// Either way the result is exact on the fp32 scores (ties to the lower index) and
// independent of scheduling.
#include "common.hpp"
#include "launch.hpp"
#include "pool.hpp"

namespace dsv4 {

typedef int v8i32 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kThreads = 256;
// 16-key tiles per wave and step: enough loads in flight per lane (the next step's tiles
// are loaded while this step's are used) within a register budget of about 80 VGPRs.
template <int KIND, int DI>
constexpr int tiles_per_step() {
  return KIND == KEY_BF16 ? (DI >= 256 ? 2 : 4) : (KIND == KEY_FP8 && DI >= 256 ? 4 : 8);
}
template <int KIND, int DI>
constexpr int keys_per_step() { return tiles_per_step<KIND, DI>() * 16 * 4; }   // 4 waves

__device__ __forceinline__ uint32_t vis_blocks(const int32_t* q_pos, int64_t row, int m, int64_t N) {
  int64_t p = q_pos[row];
  DSV4_DCHECK(p >= 0, kDbgQueryPos);
  int64_t n = (p + 1) / m;
  if (p < 0) n = 0;
  return (uint32_t)(n < N ? n : N);
}

__global__ void clear_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// LDS histograms hold two 16-bit bin counters per word (a workgroup counts fewer than
// 2^16 keys per query: kMaxIndexChunk); the flush adds them to the 32-bit row histogram.
constexpr int kHistWords = kHistBins / 2;
constexpr int64_t kMaxIndexChunk = 32768;
constexpr int64_t kXcds = 8;            // gfx950: XCDs, each with its own L2

// Writes one score and counts it in the LDS histogram of its query slot.
// kStore: the score goes to the global row here (else the caller stores it later).
template <bool kStore = true>
__device__ __forceinline__ void emit_score(float* scores, uint32_t* hist_l, int64_t row, int64_t sstride,
                                           int64_t N, int64_t key, uint32_t nvis, float v) {
  if (key >= N) return;
  bool vis = key < (int64_t)nvis;
  if constexpr (kStore) scores[row * sstride + key] = vis ? v : -INFINITY;
  if (vis) {
    const uint32_t bin = score_key(v) >> (32 - kHistBits);
    atomicAdd(&hist_l[bin >> 1], 1u << ((bin & 1u) << 4));
  }
}

template <int NT = kThreads>
__device__ __forceinline__ void flush_hist(const uint32_t* hist_l, uint32_t* hist_g, int64_t row) {
  for (int w = threadIdx.x; w < kHistWords; w += NT) {
    const uint32_t c = hist_l[w];
    if (c & 0xffffu) atomicAdd(&hist_g[row * kHistBins + 2 * w], c & 0xffffu);
    if (c >> 16) atomicAdd(&hist_g[row * kHistBins + 2 * w + 1], c >> 16);
  }
}

// ------------------------------------------------------------------ block-wide helpers
// Inclusive prefix sum over the 64 lanes of a wave: row shifts within each 16-lane row,
// then the last lane of a row is broadcast into the following rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Block-wide exclusive prefix sum for NT threads (NT / 64 waves); `tmp` holds NT / 64
// words of LDS.  Returns the exclusive prefix and writes the total to *total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = tmp[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Minimum of a 64-bit value over an NT-thread workgroup (tmp: 2 * NT / 64 words of LDS).
template <int NT>
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint32_t* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  if (lane == 0) {
    tmp[2 * wave] = (uint32_t)v;
    tmp[2 * wave + 1] = (uint32_t)(v >> 32);
  }
  __syncthreads();
  uint64_t r = ~0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t x = ((uint64_t)tmp[2 * w + 1] << 32) | tmp[2 * w];
    r = x < r ? x : r;
  }
  __syncthreads();
  return r;
}

// Minimum and maximum of 64-bit values over an NT-thread workgroup in one exchange
// (tmp: 4 * NT / 64 words of LDS).
template <int NT>
__device__ __forceinline__ void block_minmax_u64(uint64_t& mn, uint64_t& mx, uint32_t* tmp) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t a = __shfl_xor(mn, o), b = __shfl_xor(mx, o);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) {
    tmp[4 * wave] = (uint32_t)mn;
    tmp[4 * wave + 1] = (uint32_t)(mn >> 32);
    tmp[4 * wave + 2] = (uint32_t)mx;
    tmp[4 * wave + 3] = (uint32_t)(mx >> 32);
  }
  __syncthreads();
  mn = ~0ull;
  mx = 0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t a = ((uint64_t)tmp[4 * w + 1] << 32) | tmp[4 * w];
    const uint64_t b = ((uint64_t)tmp[4 * w + 3] << 32) | tmp[4 * w + 2];
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  __syncthreads();
}

// Composite selection key: the score key in the high half and the complemented block
// index in the low half, so that a larger composite is a larger score or, for equal
// scores, a lower index; the composites of different blocks are distinct, and no real
// score gives the composite 0 (which marks an empty slot).
__device__ __forceinline__ uint64_t comp_key(float s, uint32_t j) {
  return ((uint64_t)score_key(s) << 32) | (uint64_t)(~j);
}

constexpr int kRadixBits = 12;                               // digit width of the radix selections

// The need-th largest of c distinct composites get(0) .. get(c-1) (1 <= need <= the number
// of nonzero ones): radix selection from the top bit down, kRadixBits per round, over an LDS
// histogram (hbin: 1 << kRadixBits words; tmp: 2 NT / 64 words; misc: 3 words).  Exactly
// `need` composites are >= the result.  Rounds stop as soon as the digit bin holding the
// boundary is taken whole.  Every thread returns the same value.
template <int NT, class Get>
__device__ __forceinline__ uint64_t kth_largest(Get get, uint32_t c, uint32_t need, uint32_t* hbin, uint32_t* tmp, uint32_t* misc) {
  constexpr int kBins = 1 << kRadixBits;
  constexpr int BPT = kBins / NT;
  static_assert(BPT >= 1 && kBins % NT == 0, "digit bins per thread");
  const int tid = threadIdx.x;
  // The top bits that every nonzero composite shares need no round: the rounds start below
  // the highest bit in which the smallest and the largest differ (so that the first
  // round's digits spread over the histogram instead of piling onto a few bins).
  uint64_t mn = ~0ull, mx = 0ull;
  for (uint32_t f = tid; f < c; f += NT) {
    const uint64_t v = get(f);
    if (v != 0ull) {
      mn = v < mn ? v : mn;
      mx = v > mx ? v : mx;
    }
  }
  mn = block_min_u64<NT>(mn, tmp);
  mx = ~block_min_u64<NT>(~mx, tmp);
  const uint64_t diff = mn ^ mx;
  int hi = diff ? 64 - __clzll((long long)diff) : 0;         // bits [hi-1 : 0] still open
  uint64_t prefix = hi == 64 ? 0ull : (mx >> hi) << hi;
  while (true) {
    const int wd = hi < kRadixBits ? hi : kRadixBits;
    const int sh = hi - wd;
    const int nd = 1 << wd;
    for (int i = tid; i < kBins; i += NT) hbin[i] = 0u;
    __syncthreads();
    for (uint32_t f = tid; f < c; f += NT) {
      const uint64_t v = get(f);
      if (hi == 64 || (v >> hi) == (prefix >> hi)) atomicAdd(&hbin[(uint32_t)(v >> sh) & (uint32_t)(nd - 1)], 1u);
    }
    __syncthreads();
    // thread t holds digits nd-1-(BPT t + i), i = 0 .. BPT-1 (descending), so that the
    // exclusive prefix counts the composites with larger digits
    uint32_t hv[BPT];
    uint32_t tsum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int d = BPT * tid + i;
      hv[i] = d < nd ? hbin[nd - 1 - d] : 0u;
      tsum += hv[i];
    }
    uint32_t tot;
    const uint32_t ex = block_scan<NT>(tsum, tmp, &tot);
    if (ex < need && need <= ex + tsum) {
      uint32_t acc = ex;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        if (acc < need && need <= acc + hv[i]) {
          misc[0] = (uint32_t)(nd - 1 - (BPT * tid + i));
          misc[1] = acc;
          misc[2] = hv[i];
        }
        acc += hv[i];
      }
    }
    __syncthreads();
    need -= misc[1];
    prefix |= (uint64_t)misc[0] << sh;
    const bool done = misc[2] == need || sh == 0;
    hi = sh;
    __syncthreads();                                         // misc is rewritten next round
    if (done) break;
  }
  return prefix;
}

// Local selection at the end of an index workgroup (decode-shaped calls), from the chunk's
// visible scores sc[0 .. nv) and their 12-bit histogram hist16 (two 16-bit counters per
// word), both built in LDS as the scores were emitted.  The workgroup keeps whole histogram
// bins: every key in the bins from the one holding its KL-th largest score upward, or, when
// that would be more than KL keys, from the next bin up (then fewer than KL).  The kept keys
// are written as composites, in ascending key order, to out[0 .. count) and *meta receives
// {count, nv, floor (low, high words)}: every kept composite is >= floor and every omitted
// one is below it.  With nv <= KL every visible key is kept (floor 0).
// key0: index of the chunk's first key; hb: 1 << kRadixBits words of LDS (staging);
// tmp: 2 NT / 64 words; misc: 4 words.
constexpr int kLocalChunk = 4096;                            // keys per index workgroup (local selection)
constexpr size_t kMinLocalLds = 56 * 1024;                   // LDS of a local-path index workgroup
constexpr int kLocalWaves = 8;                               // waves of a local-path index workgroup
template <int NT>
__device__ __forceinline__ void local_select(const float* sc, uint32_t nv, const uint32_t* hist16, uint32_t KL, uint32_t key0,
                             uint64_t* __restrict__ out, uint4* __restrict__ meta, uint32_t* hb, uint32_t* tmp,
                             uint32_t* misc) {
  const int tid = threadIdx.x;
  if (nv <= KL) {
    for (uint32_t i = tid; i < nv; i += NT) out[i] = comp_key(sc[i], key0 + i);
    if (tid == 0) *meta = make_uint4(nv, nv, 0u, 0u);
    return;
  }
  // 1. the bin holding the KL-th largest score, the count above it and its own count
  constexpr int BPT = kHistBins / NT;
  static_assert(BPT % 2 == 0, "whole histogram words per thread");
  uint32_t cnt[BPT];
  uint32_t tsum = 0;
  static_assert((BPT / 2) % 4 == 0, "16-byte reads of the packed histogram");
#pragma unroll
  for (int i = 0; i < BPT / 2; i += 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(hist16 + tid * (BPT / 2) + i);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cnt[2 * (i + j)] = w4[j] & 0xffffu;
      cnt[2 * (i + j) + 1] = w4[j] >> 16;
      tsum += cnt[2 * (i + j)] + cnt[2 * (i + j) + 1];
    }
  }
  uint32_t total;
  const uint32_t excl = block_scan<NT>(tsum, tmp, &total);
  const uint32_t above = total - excl - tsum;               // keys in higher threads' bins
  if (above < KL && KL <= above + tsum) {
    uint32_t acc = above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {                      // (no early exit: cnt stays in registers)
      if (acc < KL && KL <= acc + cnt[i]) {
        misc[0] = tid * BPT + i;
        misc[1] = acc;
        misc[2] = cnt[i];
      }
      acc += cnt[i];
    }
  }
  __syncthreads();
  const uint32_t keep_bin = misc[1] + misc[2] <= KL ? misc[0] : misc[0] + 1;
  // 2. one pass: wave w takes keys [KPW w, KPW (w+1)), 64 consecutive keys per step (conflict-
  //    free LDS reads, all issued before they are used); kept keys are staged in LDS
  constexpr int NW = NT / kWave;
  constexpr int KPW = kLocalChunk / NW;
  constexpr int STEPS = KPW / kWave;
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t w0 = (uint32_t)wave * KPW;
  uint64_t* stage = reinterpret_cast<uint64_t*>(hb);         // KL <= (1 << kRadixBits) / 2 entries
  float v[STEPS];
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {                          // (keys past nv are ignored below)
    const uint32_t i = w0 + u * kWave + lane;
    v[u] = sc[i < nv ? i : nv - 1];
  }
  uint64_t masks[STEPS];
  uint32_t wtot = 0;
  if (w0 + KPW <= nv && keep_bin > 0) {                      // the wave's keys are all visible
    // score_key is monotone, so "key >= the bin's first key" is one float compare against
    // the smallest score of bin keep_bin (nothing is kept past the last bin)
    const uint32_t kf = keep_bin << (32 - kHistBits);
    const float thr = keep_bin >= (uint32_t)kHistBins ? INFINITY
                                                       : __uint_as_float(kf & 0x80000000u ? kf & 0x7fffffffu : ~kf);
    const bool none = keep_bin >= (uint32_t)kHistBins;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      masks[u] = __ballot(!none && v[u] >= thr);
      wtot += (uint32_t)__popcll(masks[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const uint32_t i = w0 + u * kWave + lane;
      masks[u] = __ballot(i < nv && (score_key(v[u]) >> (32 - kHistBits)) >= keep_bin);
      wtot += (uint32_t)__popcll(masks[u]);
    }
  }
  // staging offsets in wave order, so that the list is in ascending key order (the row
  // selection relies on it to compact its result without a key bitmap)
  if (lane == 0) tmp[wave] = wtot;
  __syncthreads();
  uint32_t base = 0, staged = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = tmp[w];
    base += w < wave ? x : 0u;
    staged += x;
  }
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const uint64_t mask = masks[u];
    const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (((mask >> lane) & 1ull) && pos < KL) stage[pos] = comp_key(v[u], key0 + w0 + u * kWave + lane);
    base += (uint32_t)__popcll(mask);
  }
  __syncthreads();
  DSV4_DCHECK(staged <= KL, kDbgLocalStage);
  const uint32_t count = staged < KL ? staged : KL;
  for (uint32_t j = tid; j < count; j += NT) out[j] = stage[j];
  if (tid == 0) {
    const uint64_t floor = keep_bin >= (uint32_t)kHistBins ? ~0ull : (uint64_t)(keep_bin << (32 - kHistBits)) << 32;
    *meta = make_uint4(count, nv, (uint32_t)floor, (uint32_t)(floor >> 32));
  }
}

// ------------------------------------------------------------------ fp32 keys (VALU)
__global__ __launch_bounds__(kThreads) void index_f32_kernel(
    const float* __restrict__ qi, const float* __restrict__ wi, const float* __restrict__ ki,
    const int32_t* __restrict__ q_pos, int64_t N, int64_t k_bs, int64_t Q, int HI, int DI, int m,
    float* __restrict__ scores, int64_t sstride, uint32_t* __restrict__ hist_g) {
  extern __shared__ uint32_t sm[];
  uint32_t* hist_l = sm;
  float* qs = reinterpret_cast<float*>(sm + kHistWords);
  float* ws = qs + HI * DI;
  const int64_t row = blockIdx.y;            // b * Q + q
  const int64_t b = row / Q;
  for (int i = threadIdx.x; i < kHistWords; i += kThreads) hist_l[i] = 0u;
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
  template <bool kNT>
  __device__ void load(const uint8_t* kbase, const uint8_t*, int64_t key, int g, bool ok) {
    const uint4* p = reinterpret_cast<const uint4*>(kbase + key * (DI * 2) + g * (DI / 2));
#pragma unroll
    for (int c = 0; c < KS; ++c) w[c] = ok ? load_key<kNT>(p + c) : make_uint4(0, 0, 0, 0);
  }
  __device__ bf16x8 op(int c) const { return bit_cast_to<bf16x8>(w[c]); }
};

template <int DI>
struct KeyTile<KEY_MXFP4, DI> {
  static constexpr int KS = DI / 32;
  uint32_t w[KS];
  uint32_t sc;   // up to 2 scale bytes for this lane's dims
  template <bool kNT>
  __device__ void load(const uint8_t* kbase, const uint8_t* sbase, int64_t key, int g, bool ok) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(kbase + key * (DI / 2) + g * (DI / 8));
    if constexpr (KS % 4 == 0) {          // 16-byte aligned: whole dwordx4 loads
#pragma unroll
      for (int c = 0; c < KS; c += 4) {
        const uint4 v = ok ? load_key<kNT>(reinterpret_cast<const uint4*>(p + c)) : make_uint4(0, 0, 0, 0);
        w[c] = v.x; w[c + 1] = v.y; w[c + 2] = v.z; w[c + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < KS; ++c) w[c] = ok ? load_key<kNT>(p + c) : 0u;
    }
    const uint8_t* s = sbase + key * (DI / 32) + (g * (DI / 4)) / 32;
    if constexpr (DI == 256) sc = ok ? load_key<kNT>(s) | (load_key<kNT>(s + 1) << 8) : 0x7f7fu;
    else sc = ok ? load_key<kNT>(s) : 0x7fu;
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

// MXFP4 keys for the FP4 x FP4 product: the raw code words and scale bytes feed the
// scaled MFMA directly (lane g's 32-element block c is words 4c .. 4c+3, scale byte c).
template <int DI>
struct KeyTile<KEY_MXFP4_Q4, DI> : KeyTile<KEY_MXFP4, DI> {};

template <int DI>
struct KeyTile<KEY_FP8, DI> {
  static constexpr int KS = DI / 32;
  uint2 w[KS];
  template <bool kNT>
  __device__ void load(const uint8_t* kbase, const uint8_t*, int64_t key, int g, bool ok) {
    const uint2* p = reinterpret_cast<const uint2*>(kbase + key * DI + g * (DI / 4));
#pragma unroll
    for (int c = 0; c < KS; ++c) w[c] = ok ? load_key<kNT>(p + c) : make_uint2(0, 0);
  }
  __device__ long op(int c) const { return __builtin_bit_cast(long, w[c]); }
};

// The pooling of a decode step's newest block inside the indexer launch (see IndexPool).
// Grid rows at and past index_rows run the K|V rows' job; in the index grid, the wave
// whose keys include the pooled row pools that sequence's indexer key on its own (a wave
// of lanes, lpr2 * spb2 <= 64: no workgroup barrier) and stores it before any load of it.
struct PoolDev {
  int on;
  int index_rows;
  int kv_fp8;
  int m;
  int64_t nblk;                  // sequences (one block each)
  const uint16_t* x2;
  int64_t x2_bs;                 // elements between sequences of x2
  const float* gate;
  const float* bias;
  int64_t row;
  int lpr2, spb2;
  pool::Job kv;
};

// QTW query tiles (QTW * 16/HI queries) per workgroup: every key tile loaded is used by
// all of them (QTW > 1 when there are many queries, e.g. a prefill chunk).
// kLocal (decode-shaped calls, QTW = 1, chunk <= kLocalChunk): the workgroup also keeps its
// chunk's scores in LDS and ends with a local selection of each query's klocal best keys
// (cand_loc [rows][nch][klocal] composites, meta_loc [rows][nch]); the row histogram in
// hist_g is not used.
template <int KIND, int DI, int HI, int QTW, bool kNT, bool kLocal, int NW = 4>
__global__ __launch_bounds__(NW * kWave) void index_mfma_kernel(
    const uint8_t* __restrict__ qi, const uint8_t* __restrict__ qsc, const float* __restrict__ wi,
    const uint8_t* ki, const uint8_t* ksc, const int32_t* __restrict__ q_pos, int64_t N,
    int64_t k_bs, int64_t Q, int m, int64_t chunk, float* __restrict__ scores, int64_t sstride,
    uint32_t* __restrict__ hist_g, uint64_t* __restrict__ cand_loc, uint4* __restrict__ meta_loc, int klocal,
    int nch, PoolDev pd) {
  // (ki and ksc carry no restrict: with pooling, a row of them is written below)
  constexpr int QPT = 16 / HI;          // queries per 16-row MFMA tile
  constexpr int KS = DI / 32;
  constexpr int GPQ = HI / 4;           // lane groups per query slot
  constexpr int NTH = NW * kWave;       // threads
  static_assert(!kLocal || QTW == 1, "local selection: one query tile per workgroup");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  // LDS: [QTW * QPT][kHistWords] histograms (kLocal: [min(Q, QPT)]), with kLocal then the
  // scores [min(Q, QPT)][chunk] and the selection's scratch.  A pooling workgroup uses the
  // start of the same space for its states (the launch sizes it for both).
  extern __shared__ uint32_t hist_l[];
  float* const sc_l = reinterpret_cast<float*>(hist_l + (kLocal ? (Q < QPT ? Q : QPT) : QTW * QPT) * kHistWords);
  uint32_t* const selb = reinterpret_cast<uint32_t*>(sc_l + (kLocal ? (Q < QPT ? Q : QPT) * chunk : 0));

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  if (pd.on && (int)blockIdx.y >= pd.index_rows) {          // the K|V rows' pooling job
    const int64_t wg = (int64_t)(blockIdx.y - pd.index_rows) * gridDim.x + blockIdx.x;
    float* const pool_part = reinterpret_cast<float*>(hist_l);
    if (wg < pd.kv.grid) {
      if (pd.kv_fp8)
        pool::compress_body<uint16_t, 4>(reinterpret_cast<const uint16_t*>(pd.kv.x), pd.gate, pd.bias, pd.m, pd.kv.C,
                                         pd.m, 1, pd.nblk, pd.kv.x_bs, pd.kv.y_bs, pd.kv.y, pd.kv.ysc, pd.kv.lpr,
                                         pd.kv.spb, pd.kv.bpw, pd.kv.cs, wg, pool_part);
      else
        pool::compress_body<uint16_t, 1>(reinterpret_cast<const uint16_t*>(pd.kv.x), pd.gate, pd.bias, pd.m, pd.kv.C,
                                         pd.m, 1, pd.nblk, pd.kv.x_bs, pd.kv.y_bs, pd.kv.y, pd.kv.ysc, pd.kv.lpr,
                                         pd.kv.spb, pd.kv.bpw, pd.kv.cs, wg, pool_part);
    }
    return;
  }
  const int64_t QT = (Q + QPT - 1) / QPT;
  const int64_t QG = (QT + QTW - 1) / QTW;
  const int64_t b = blockIdx.y / QG, qt0 = (blockIdx.y % QG) * QTW;
  // key range of this workgroup; the first step's key tiles are loaded before anything
  // else so that their latency overlaps the query loads below
  const uint8_t* kbase;
  const uint8_t* sbase = nullptr;
  if constexpr (KIND == KEY_BF16) kbase = ki + b * k_bs * DI * 2;
  else if constexpr (KIND == KEY_FP8) kbase = ki + b * k_bs * DI;
  else {
    kbase = ki + b * k_bs * (DI / 2);
    sbase = ksc + b * k_bs * (DI / 32);
  }
  // (eight waves take half the tiles per step, so that a step covers the same keys)
  constexpr int TPW = QTW == 1 ? (NW == 8 && tiles_per_step<KIND, DI>() > 1 ? tiles_per_step<KIND, DI>() / 2
                                                                            : tiles_per_step<KIND, DI>())
                               : (KIND == KEY_FP8 && NW == 4 ? 4 : 2);
  constexpr int KPS = TPW * 16 * NW;
  constexpr int E = GPQ < TPW ? GPQ : TPW;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  int64_t c1 = c0 + chunk;
  if (c1 > N) c1 = N;
  const int64_t klast = c1 - 1;
  if constexpr (KIND == KEY_MXFP4 || KIND == KEY_MXFP4_Q4) {
    // the pooled indexer key of this sequence, by the wave that loads it, before its loads
    // (lpr2 * spb2 <= 64, both powers of two: the states combine inside the wave, without
    // LDS or a barrier)
    if (pd.on && pd.row >= c0 && pd.row < c1 && wave == (int)(((pd.row - c0) % KPS) / (TPW * 16))) {
      pool::compress_body<uint16_t, 3>(pd.x2 + b * pd.x2_bs, pd.gate + b * pd.m, pd.bias, pd.m, DI, pd.m, 1, 1, 0, 0,
                                       const_cast<uint8_t*>(kbase) + pd.row * (DI / 2),
                                       const_cast<uint8_t*>(sbase) + pd.row * (DI / 32), pd.lpr2, pd.spb2, 1, 1, 0,
                                       nullptr, nullptr, 0.f, lane);
      wait_vmcnt0();
    }
    asm volatile("" ::: "memory");
  }
  KeyTile<KIND, DI> cur[TPW], nxt[TPW];
  int64_t base = c0 + wave * (TPW * 16);
  if (base < c1) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int64_t key = base + u * 16 + col;
      cur[u].template load<kNT>(kbase, sbase, key < klast ? key : klast, g, true);
    }
  }

  int nq[QTW];
  int nslots = 0;
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int64_t left = Q - (qt0 + t) * QPT;
    nq[t] = left <= 0 ? 0 : (left < QPT ? (int)left : QPT);
    nslots += kLocal ? nq[t] : (nq[t] > 0 ? QPT : 0);
  }
  for (int i = threadIdx.x; i < nslots * kHistWords; i += NTH) hist_l[i] = 0u;
  // kLocal: the visible keys of each query of the tile, for the epilogue (loaded here, where
  // the latency is hidden behind the first key loads)
  __shared__ uint32_t nvis_ep[kLocal ? QPT : 1];
  if constexpr (kLocal) {
    if ((int)threadIdx.x < nq[0]) nvis_ep[threadIdx.x] = vis_blocks(q_pos, b * Q + qt0 * QPT + threadIdx.x, m, N);
  }

  // A operands: query rows (row = lane % 16 = qslot * HI + head) of each query tile
  const int qs_a = col / HI, h_a = col % HI;
  uint4 qa16[QTW][KS];   // bf16 queries
  uint2 qa8[QTW][KS];    // fp8 queries
  constexpr int KS4 = DI / 128 > 0 ? DI / 128 : 1;   // FP4 x FP4: 128-deep MFMA steps
  uint4 qa4[QTW][KS4];   // MXFP4 query codes (32 per lane and step)
  uint32_t qs4[QTW];     // their scale bytes (byte c: step c)
  // epilogue: accumulator row 4g+i -> (slot (4g+i)/HI, head (4g+i)%HI)
  const int qs_c = (4 * g) / HI;
  const int esel = g % GPQ;              // this lane's tile within a group of E emitted together
  float wv[QTW][4];
  uint32_t nvis[QTW];
  int64_t row_c[QTW];
  bool owner[QTW];
#pragma unroll
  for (int t = 0; t < QTW; ++t) {
    const int64_t qbase = b * Q + (qt0 + t) * QPT;
    const bool qa_ok = qs_a < nq[t];
    const int64_t qrow_a = (qa_ok ? qbase + qs_a : b * Q) * HI + h_a;
    if constexpr (KIND == KEY_MXFP4_Q4) {
      const uint4* p = reinterpret_cast<const uint4*>(qi + qrow_a * (DI / 2) + g * (DI / 8));
#pragma unroll
      for (int c = 0; c < KS4; ++c) qa4[t][c] = qa_ok ? p[c] : make_uint4(0, 0, 0, 0);
      const uint8_t* sp = qsc + qrow_a * (DI / 32) + g * KS4;
      uint32_t sv = 0;
#pragma unroll
      for (int c = 0; c < KS4; ++c) sv |= (uint32_t)sp[c] << (8 * c);
      qs4[t] = qa_ok ? sv : 0x7f7f7f7fu;
    } else if constexpr (KIND == KEY_FP8) {
      const uint2* p = reinterpret_cast<const uint2*>(qi + qrow_a * DI + g * (DI / 4));
#pragma unroll
      for (int c = 0; c < KS; ++c) qa8[t][c] = qa_ok ? p[c] : make_uint2(0, 0);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(qi + (qrow_a * DI + g * (DI / 4)) * 2);
#pragma unroll
      for (int c = 0; c < KS; ++c) qa16[t][c] = qa_ok ? p[c] : make_uint4(0, 0, 0, 0);
    }
    const bool qc_ok = qs_c < nq[t];
    row_c[t] = qc_ok ? qbase + qs_c : b * Q;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = qc_ok ? wi[row_c[t] * HI + ((4 * g + i) % HI)] : 0.f;
    nvis[t] = qc_ok ? vis_blocks(q_pos, row_c[t], m, N) : 0u;
    owner[t] = qc_ok && esel < E;
  }
  __syncthreads();

  // Each wave takes TPW consecutive 16-key tiles per step; the next step's tiles are
  // loaded before this step's are used.  Key indices past the range are clamped to its
  // last key, so loads never branch; only the score write is guarded.  Two steps per
  // iteration with the tile buffers' roles swapped, so that no buffer is copied.
  auto step = [&](KeyTile<KIND, DI>(&cu)[TPW], KeyTile<KIND, DI>(&nx)[TPW], const int64_t base) {
    const int64_t nb = base + KPS;
    if (nb < c1) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int64_t key = nb + u * 16 + col;
        nx[u].template load<kNT>(kbase, sbase, key < klast ? key : klast, g, true);
      }
    }
    // After the head reduction the GPQ lanes of a query slot hold the same score, so E
    // consecutive tiles are emitted together: lane group e of the slot writes tile u + e.
#pragma unroll
    for (int u = 0; u < TPW; u += E) {
#pragma unroll
      for (int t = 0; t < QTW; ++t) {
        float vs = 0.f;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (KIND == KEY_MXFP4_Q4) {
#pragma unroll
            for (int c = 0; c < KS4; ++c) {
              const auto& kt = cu[u + j];
              const v8i32 av = {(int)qa4[t][c].x, (int)qa4[t][c].y, (int)qa4[t][c].z, (int)qa4[t][c].w, 0, 0, 0, 0};
              const v8i32 bv = {(int)kt.w[4 * c], (int)kt.w[4 * c + 1], (int)kt.w[4 * c + 2], (int)kt.w[4 * c + 3],
                                0, 0, 0, 0};
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0,
                                                                      (int)((qs4[t] >> (8 * c)) & 0xffu), 0,
                                                                      (int)((kt.sc >> (8 * c)) & 0xffu));
            }
          } else if constexpr (KIND == KEY_FP8 && DI >= 128) {
            // fp8 x fp8 on the scaled 16x16x128 MFMA with unit scales (E8M0 127): the fp8
            // 16x16x32 form runs at the bf16 rate on gfx950, this one at the fp8 rate.  A
            // lane's 32 codes of 128-dim block c are its k-step words 4c .. 4c+3 (the same
            // dims for the query and the key operand).
#pragma unroll
            for (int c = 0; c < DI / 128; ++c) {
              const auto& kt = cu[u + j];
              const uint2* qw = qa8[t] + 4 * c;
              const v8i32 av = {(int)qw[0].x, (int)qw[0].y, (int)qw[1].x, (int)qw[1].y,
                                (int)qw[2].x, (int)qw[2].y, (int)qw[3].x, (int)qw[3].y};
              const v8i32 bv = {(int)kt.w[4 * c].x, (int)kt.w[4 * c].y, (int)kt.w[4 * c + 1].x,
                                (int)kt.w[4 * c + 1].y, (int)kt.w[4 * c + 2].x, (int)kt.w[4 * c + 2].y,
                                (int)kt.w[4 * c + 3].x, (int)kt.w[4 * c + 3].y};
              acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
            }
          } else {
#pragma unroll
            for (int c = 0; c < KS; ++c) {
              if constexpr (KIND == KEY_FP8)
                acc = mfma_fp8(__builtin_bit_cast(long, qa8[t][c]), cu[u + j].op(c), acc);
              else acc = mfma_bf16(bit_cast_to<bf16x8>(qa16[t][c]), cu[u + j].op(c), acc);
            }
          }
          float v = wv[t][0] * fmaxf(acc[0], 0.f);
          v = fmaf(wv[t][1], fmaxf(acc[1], 0.f), v);
          v = fmaf(wv[t][2], fmaxf(acc[2], 0.f), v);
          v = fmaf(wv[t][3], fmaxf(acc[3], 0.f), v);
          if constexpr (GPQ >= 2) v = add_xor16(v);
          if constexpr (GPQ >= 4) v = add_xor32(v);
          vs = (j == esel) ? v : vs;
        }
        const int64_t key = base + (u + esel) * 16 + col;
        if (owner[t] && key < c1) {
          emit_score<!kLocal>(scores, hist_l + (t * QPT + qs_c) * kHistWords, row_c[t], sstride, N, key, nvis[t],
                              vs);
          if constexpr (kLocal) sc_l[qs_c * chunk + (key - c0)] = key < (int64_t)nvis[t] ? vs : -INFINITY;
        }
      }
    }
  };
  for (; base < c1; base += 2 * KPS) {
    step(cur, nxt, base);
    if (base + KPS < c1) step(nxt, cur, base + KPS);
  }
  __syncthreads();
  if constexpr (kLocal) {
    // each query's klocal best keys of this chunk; then its scores go to the global row in
    // 16-byte stores (they are read back only to widen a chunk, or for out_score)
    for (int s = 0; s < nq[0]; ++s) {
      const int64_t row = b * Q + qt0 * QPT + s;
      int64_t nv = (int64_t)nvis_ep[s] - c0;
      nv = nv < 0 ? 0 : (nv > c1 - c0 ? c1 - c0 : nv);
      const int64_t slot = row * nch + blockIdx.x;
      local_select<NTH>(sc_l + s * chunk, (uint32_t)nv, hist_l + s * kHistWords, (uint32_t)klocal, (uint32_t)c0,
                             cand_loc + slot * klocal, meta_loc + slot, selb, selb + (1 << kRadixBits),
                             selb + (1 << kRadixBits) + 2 * NTH / kWave);
      const float* src = sc_l + s * chunk;
      float* dst = scores + row * sstride + c0;
      const int64_t nk = c1 - c0;                            // c0 and the row stride are multiples of 64
      for (int64_t i = (int64_t)threadIdx.x * 4; i < nk; i += NTH * 4) {
        if (i + 4 <= nk) *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(src + i);
        else for (int64_t j = i; j < nk; ++j) dst[j] = src[j];
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int t = 0; t < QTW; ++t)
      for (int s = 0; s < nq[t]; ++s)
        flush_hist<NTH>(hist_l + (t * QPT + s) * kHistWords, hist_g, b * Q + (qt0 + t) * QPT + s);
  }
}

// ------------------------------------------------------------------ selection
// Threshold bin of a row: the bin b* with #(bin > b*) < kk <= #(bin >= b*).  Every thread
// of an NT-thread workgroup takes kHistBins / NT consecutive bins; the result goes to
// misc[0] (bin) and misc[1] (#keys above it).
template <int NT>
__device__ __forceinline__ void threshold_bin(const uint32_t* __restrict__ hr, uint32_t kk, uint32_t* tmp,
                                              uint32_t* misc) {
  constexpr int BPT = kHistBins / NT;
  uint32_t hv[BPT];
  uint32_t tsum = 0;
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(hr + threadIdx.x * BPT + i);
    hv[i] = v.x; hv[i + 1] = v.y; hv[i + 2] = v.z; hv[i + 3] = v.w;
    tsum += v.x + v.y + v.z + v.w;
  }
  uint32_t total;
  const uint32_t excl = block_scan<NT>(tsum, tmp, &total);
  const uint32_t above = total - excl - tsum;                // keys in higher threads' bins
  if (above < kk && kk <= above + tsum) {
    uint32_t acc = above;
    for (int i = BPT - 1; i >= 0; --i) {
      if (acc + hv[i] >= kk) {
        misc[0] = threadIdx.x * BPT + i;
        misc[1] = acc;
        break;
      }
      acc += hv[i];
    }
  }
  __syncthreads();
}

// Selection, pass 1 (all rows x key ranges of KEYS keys): keys above the threshold bin
// get their bit in the row's key bitmap (whole 32-bit words, plain stores); keys inside
// the bin are appended to this range's own slice of the candidate buffer as composite
// keys (score key << 32 | ~index: equal scores order the lower index first), and the
// range's candidate count is stored.
constexpr int kScanThreads = 256;
constexpr int kScanKeys = 2048;                              // range of few-row calls: 2 float4 per thread
constexpr int kScanKeysMany = 8192;                          // range of calls with >= kManyRows rows
constexpr int64_t kManyRows = 256;
// Many rows (a prefill chunk) fill the GPU with long ranges, which read the row's histogram
// for the threshold 4x less often per key; few long rows need the shorter ranges to have
// enough workgroups.
inline int64_t scan_keys(int64_t rows) { return rows >= kManyRows ? kScanKeysMany : kScanKeys; }
constexpr int kFinThreads = 1024;
constexpr int kLdsBitmapKeys = 1 << 18;                      // bitmap kept in LDS by pass 2
constexpr int kLdsBitmapKeysSmall = 1 << 17;                 // ... in a workgroup that fits twice on a CU
constexpr int kCandCap = 4096;                               // candidates staged in LDS by pass 2

// Selection, pass 0 (one workgroup per row): the row's threshold bin and the count of keys
// above it, from its histogram, recorded for the scan ranges and the finish pass (each scan
// range then reads two words instead of the 16 KB histogram).
__global__ __launch_bounds__(kScanThreads) void select_threshold_kernel(const uint32_t* __restrict__ hist_g,
                                                                        uint32_t* __restrict__ thr,
                                                                        const int32_t* __restrict__ q_pos, int64_t N,
                                                                        int m, int k) {
  __shared__ uint32_t tmp[kScanThreads / kWave];
  __shared__ uint32_t misc[4];
  const int64_t row = blockIdx.x;
  const uint32_t n = vis_blocks(q_pos, row, m, N);
  const uint32_t kk = (uint32_t)k < n ? (uint32_t)k : n;
  if (kk == 0) return;                     // (the passes below return before reading it)
  threshold_bin<kScanThreads>(hist_g + row * kHistBins, kk, tmp, misc);
  if (threadIdx.x == 0) {
    thr[row * 2] = misc[0];
    thr[row * 2 + 1] = misc[1];
  }
}

template <int KEYS>
__global__ __launch_bounds__(kScanThreads) void select_scan_kernel(
    const float* __restrict__ scores, uint32_t* __restrict__ bitmap_g, uint64_t* __restrict__ cand_g,
    uint32_t* __restrict__ ccount, const uint32_t* __restrict__ thr, const int32_t* __restrict__ q_pos, int64_t N,
    int64_t sstride, int64_t words, int m, int k) {
  __shared__ uint32_t misc[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = blockIdx.y;
  const uint32_t n = vis_blocks(q_pos, row, m, N);
  const uint32_t kk = (uint32_t)k < n ? (uint32_t)k : n;
  const int64_t c0 = (int64_t)blockIdx.x * KEYS;
  const int64_t nch = gridDim.x;
  if (kk == 0 || c0 >= (int64_t)n) {
    if (tid == 0) ccount[row * nch + blockIdx.x] = 0u;
    return;
  }
  // issue the score loads first; the threshold is read while they are in flight
  const float* sc = scores + row * sstride + c0;
  const int64_t c1 = (c0 + KEYS < (int64_t)n ? c0 + KEYS : (int64_t)n) - c0;   // keys in range
  constexpr int IT = KEYS / (4 * kScanThreads);
  float4 v[IT];
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int64_t kb = (int64_t)(u * kScanThreads + tid) * 4;
    if (kb < c1) {
      const uint4 x = load_stream(reinterpret_cast<const uint4*>(sc) + u * kScanThreads + tid);   // read once
      v[u] = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    } else {
      v[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
  }
  if (tid == 0) misc[2] = 0u;
  // the row's threshold bin, recorded by select_threshold_kernel (a uniform load)
  const uint32_t tbin = *reinterpret_cast<const __attribute__((address_space(4))) uint32_t*>(
      reinterpret_cast<uintptr_t>(thr + row * 2));
  __syncthreads();                         // (misc[2] is cleared before any range count)

  uint32_t* bm = bitmap_g + row * words + c0 / 32;
  uint64_t* cs = cand_g + row * N + c0;
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int64_t kb = (int64_t)(u * kScanThreads + tid) * 4;   // this lane's 4 keys
    const float e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t nib = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sk = score_key(e4[e]);
      const uint32_t bin = sk >> (32 - kHistBits);
      const bool in = kb + e < c1;
      if (in && bin > tbin) nib |= 1u << e;
      const bool isc = in && bin == tbin;
      const uint64_t mask = __ballot(isc);
      if (mask) {
        const int leader = __ffsll((unsigned long long)mask) - 1;
        uint32_t base = 0;
        if (lane == leader) base = atomicAdd(&misc[2], (uint32_t)__popcll(mask));
        base = __builtin_amdgcn_readlane(base, leader);          // leader is the same in every lane
        if (isc) {
          const uint32_t f = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          cs[f] = ((uint64_t)sk << 32) | (uint64_t)(~(uint32_t)(c0 + kb + e));
        }
      }
    }
    // a bitmap word is the nibbles of 8 consecutive lanes, OR-ed by DPP moves: lane ^ 1 and
    // lane ^ 2 (quad permutes), then the mirrored lane of the other quad (row_half_mirror)
    uint32_t wv = nib << (4 * (lane & 7));
    wv |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wv, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
    wv |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wv, 0x4E, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
    wv |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wv, 0x141, 0xf, 0xf, false);   // row_half_mirror
    if ((lane & 7) == 0 && kb < c1) bm[kb / 32] = wv;
  }
  __syncthreads();
  if (tid == 0) ccount[row * nch + blockIdx.x] = misc[2];
}

// Selection, pass 2 (one workgroup per row): the threshold, the per-range candidate
// counts and the row's bitmap are loaded in one round, the candidates (gathered from the
// range slices) in a second; a radix select (kRadixBits-bit digits below the histogram
// prefix) finds the kk - #(bin > b*) largest candidates, their bits are added to the
// bitmap, and the bitmap is compacted into ascending indices followed by -1 padding.
// LK > 0: the row's bitmap is copied into LDS (N <= LK keys; LK = 2^17 keeps the LDS under
// 80 KB, so that two rows' workgroups share a CU); LK = 0: it stays in the workspace.
template <int LK>
__global__ __launch_bounds__(kFinThreads) __attribute__((amdgpu_waves_per_eu(8))) void select_finish_kernel(
    const float* __restrict__ scores, uint32_t* __restrict__ bitmap_g, const uint64_t* __restrict__ cand_g,
    const uint32_t* __restrict__ ccount, const uint32_t* __restrict__ thr, const int32_t* __restrict__ q_pos,
    int64_t N, int64_t sstride, int64_t words, int m, int k, int nch, int64_t rkeys, int32_t* __restrict__ out_idx,
    float* __restrict__ out_score) {
  constexpr int NT = kFinThreads;
  constexpr int kBins = 1 << kRadixBits;
  constexpr int BPT = kBins / NT;
  static_assert(BPT >= 1 && kBins % NT == 0, "digit bins per thread");
  constexpr bool kLdsBits = LK > 0;
  __shared__ uint32_t bits_l[kLdsBits ? LK / 32 : 1];
  __shared__ uint64_t cand_l[kCandCap];
  __shared__ uint32_t pre[NT + 1];                           // candidate offsets of the ranges
  __shared__ uint32_t hbin[kBins];
  __shared__ uint32_t tmp[NT / kWave];
  __shared__ uint32_t misc[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t n = vis_blocks(q_pos, row, m, N);
  const uint32_t kk = (uint32_t)k < n ? (uint32_t)k : n;
  const int64_t wn = ((int64_t)n + 31) / 32;                 // bitmap words in use
  int32_t* orow = out_idx + row * k;
  float* srow = out_score ? out_score + row * k : nullptr;
  const float* sc = scores + row * sstride;
  uint32_t* gbits = bitmap_g + row * words;
  if (kk == 0) {
    for (int p = tid; p < k; p += NT) {
      orow[p] = -1;
      if (srow) srow[p] = -INFINITY;
    }
    return;
  }
  // round 1: threshold, range counts (the first NT ranges), bitmap.  Every value read back
  // from the workspace is clamped to what pass 1 can have written (a range holds at most
  // its own keys; the count above the threshold bin is below kk), so that a wrong value
  // can only give a wrong selection, never an access outside the row's slices.
  const int nrange = (int)(((int64_t)n + rkeys - 1) / rkeys);
  auto range_count = [&](int64_t r) -> uint32_t {
    const uint32_t c_ = ccount[row * nch + r];
    const int64_t keys = (int64_t)n - r * rkeys < rkeys ? (int64_t)n - r * rkeys : rkeys;
    DSV4_DCHECK((int64_t)c_ <= keys, kDbgRangeCount);
    return c_ < (uint64_t)keys ? c_ : (uint32_t)keys;
  };
  uint2 th = *reinterpret_cast<const uint2*>(thr + row * 2);
  DSV4_DCHECK(th.x < (uint32_t)kHistBins && th.y < kk, kDbgThreshold);
  th.x &= kHistBins - 1;
  if (th.y > kk) th.y = kk;
  const uint32_t cnt0 = tid < nrange ? range_count(tid) : 0u;
  if constexpr (kLdsBits) {
    for (int64_t w = (int64_t)tid * 4; w < wn; w += (int64_t)NT * 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(gbits + w);   // rows are 16-byte padded
      *reinterpret_cast<uint4*>(bits_l + w) = x;
    }
  }
  // candidate offsets per range (more than NT ranges are summed in rounds)
  uint32_t run = 0;
  for (int r0 = 0; r0 < nrange; r0 += NT) {
    const uint32_t cnt = r0 == 0 ? cnt0 : (r0 + tid < nrange ? range_count(r0 + tid) : 0u);
    uint32_t tot;
    const uint32_t ex = block_scan<NT>(cnt, tmp, &tot);
    if (r0 + tid < nrange && r0 + tid < NT) pre[r0 + tid] = run + ex;
    run += tot;
  }
  if (tid == 0) pre[nrange < NT ? nrange : NT] = run;
  __syncthreads();
  const uint32_t c = run;
  // candidate f -> its range (binary search over the offsets; at most NT ranges are
  // indexed this way, beyond that the tail ranges are searched linearly from there)
  auto cand_at = [&](uint32_t f) -> uint64_t {
    int lo = 0, hi = (nrange < NT ? nrange : NT) - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= f) lo = mid;
      else hi = mid - 1;
    }
    uint32_t base = pre[lo];
    int64_t r = lo;
    if (r == NT - 1 && nrange > NT) {                         // rare: very long rows
      uint32_t cnt = range_count(r);
      while (f >= base + cnt && r + 1 < nrange) {
        base += cnt;
        ++r;
        cnt = range_count(r);
      }
    }
    // f < c = the sum of the clamped counts, so f - base lies inside range r's slice
    return cand_g[row * N + r * rkeys + (f - base)];
  };
  // round 2: candidates into LDS
  {
    constexpr int kPer = kCandCap / NT;
    uint64_t vals[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t f = tid + u * NT;
      vals[u] = f < c ? cand_at(f) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t f = tid + u * NT;
      if (f < c) cand_l[f] = vals[u];
    }
  }
  __syncthreads();
  auto cand = [&](uint32_t f) -> uint64_t { return f < (uint32_t)kCandCap ? cand_l[f] : cand_at(f); };

  // radix select among the candidates: composites >= tsel are taken
  uint64_t tsel = 0;
  uint32_t need = kk - th.y;
  if (need < c) {
    uint64_t prefix = (uint64_t)th.x << (64 - kHistBits);
    int hi = 64 - kHistBits;                                 // bits [hi-1 : 0] still open
    while (true) {
      const int wd = hi < kRadixBits ? hi : kRadixBits;
      const int sh = hi - wd;
      for (int i = tid; i < kBins; i += NT) hbin[i] = 0u;
      __syncthreads();
      for (uint32_t f = tid; f < c; f += NT) {
        const uint64_t comp = cand(f);
        if ((comp >> hi) == (prefix >> hi)) atomicAdd(&hbin[(comp >> sh) & ((1u << wd) - 1u)], 1u);
      }
      __syncthreads();
      // thread t holds digits nd-1-(BPT t + i), i = 0 .. BPT-1 (descending), so that the
      // exclusive prefix counts the candidates with larger digits
      const int nd = 1 << wd;
      uint32_t hv[BPT];
      uint32_t tsum = 0;
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        const int d = BPT * tid + i;
        hv[i] = d < nd ? hbin[nd - 1 - d] : 0u;
        tsum += hv[i];
      }
      uint32_t tot;
      const uint32_t ex = block_scan<NT>(tsum, tmp, &tot);
      if (ex < need && need <= ex + tsum) {
        uint32_t acc = ex;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if (acc < need && need <= acc + hv[i]) {
            misc[0] = (uint32_t)(nd - 1 - (BPT * tid + i));
            misc[1] = acc;
            misc[2] = hv[i];
          }
          acc += hv[i];
        }
      }
      __syncthreads();
      need -= misc[1];
      prefix |= (uint64_t)misc[0] << sh;
      const bool done = misc[2] == need || sh == 0;
      hi = sh;
      if (done) break;
    }
    tsel = prefix;
  }
  uint32_t* bits = kLdsBits ? bits_l : gbits;
  for (uint32_t f = tid; f < c; f += NT) {
    const uint64_t comp = cand(f);
    const uint32_t j = ~(uint32_t)comp;
    DSV4_DCHECK(comp < tsel || j < n, kDbgCandIndex);
    if (comp >= tsel && j < n) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __threadfence_block();
  __syncthreads();

  // compaction: thread t takes 8 consecutive words (256 keys) per round
  uint32_t base_off = 0;
  for (int64_t r0 = 0; r0 < wn; r0 += 8 * NT) {
    const int64_t w0 = r0 + (int64_t)tid * 8;
    uint32_t wv[8];
    if (kLdsBits && w0 + 8 <= wn) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(bits + w0);
      const uint4 x1 = *reinterpret_cast<const uint4*>(bits + w0 + 4);
      wv[0] = x0.x; wv[1] = x0.y; wv[2] = x0.z; wv[3] = x0.w;
      wv[4] = x1.x; wv[5] = x1.y; wv[6] = x1.z; wv[7] = x1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (kLdsBits) wv[i] = w0 + i < wn ? bits[w0 + i] : 0u;
        else wv[i] = w0 + i < wn ? __hip_atomic_load(&bits[w0 + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
      }
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += __popc(wv[i]);
    uint32_t rtot;
    uint32_t off = base_off + block_scan<NT>(cnt, tmp, &rtot);
    for (int i = 0; i < 8; ++i) {
      uint32_t b_ = wv[i];
      while (b_) {
        const int bpos = __ffs(b_) - 1;
        b_ &= b_ - 1;
        const int64_t j = (w0 + i) * 32 + bpos;
        if (off < (uint32_t)k) {
          orow[off] = (int32_t)j;
          if (srow) srow[off] = sc[j];
        }
        ++off;
      }
    }
    base_off += rtot;
  }
  for (int64_t p = (int64_t)base_off + tid; p < k; p += NT) {
    orow[p] = -1;
    if (srow) srow[p] = -INFINITY;
  }
}

// ---------------------------------------------------------------- local-candidate selection
// Pass 2 of decode-shaped calls, one workgroup per row (N <= kLdsBitmapKeys).  Every chunk
// kept whole histogram bins of its scores (all keys at or above its floor composite); the
// kept composites are loaded (eight slots per thread, held in registers) and the kk-th
// largest of them is found by radix selection.  A chunk that omitted keys can hide further
// winners only if its floor lies above that threshold; the omitted keys of such a chunk that
// lie above the threshold are added from the stored scores and the threshold is taken again
// (it can only rise, so no other chunk is affected).  If they do not fit in LDS, the whole
// row is selected from the stored scores instead.  The result, ascending indices of the exact
// top-kk of the fp32 scores, is compacted straight from the slots when no chunk was widened
// (the chunks' lists are in ascending key order), else through an LDS key bitmap.
constexpr int kLocalCap = 8192;          // staged candidate slots per row (nch * klocal)
constexpr int kExpCap = 4096;            // candidates added from chunks with hidden keys
constexpr int kLocalKeep = 64;           // most candidates a chunk keeps
constexpr int kMaxLocalChunks = 512;     // chunks per row on the local path
// threads of a finish workgroup (measured: 1024 threads 14.6 us per decode call, 512 17.1,
// 256 26.5; the work per thread, not the barriers, dominates)
constexpr int kLocalFinThreads = 1024;
// digit width of the finish's selection (4 bins per thread: one 16-byte LDS read)
constexpr int kLocalRadixBits = 12;

// kth_largest over values held in registers plus a list in LDS: thread t holds v[u] (0 for an
// empty slot) and the composites ext[0 .. next) are read from LDS.  Same contract and result
// as kth_largest.  Each round takes three barriers: the digit histogram (4 bins per thread,
// one 16-byte read) is scanned within each wave, the waves' totals are added from LDS by
// every thread, and the histogram of the next round is a second buffer cleared meanwhile.
// hbin2: 2 << RB words; tmp: 4 NT / 64 words; misc: 3 words.
template <int NT, int SPT, int RB>
__device__ __forceinline__ uint64_t kth_largest_regs(const uint64_t (&v)[SPT], const uint64_t* ext, uint32_t next,
                                                     uint32_t need, uint32_t* hbin2, uint32_t* tmp, uint32_t* misc) {
  constexpr int kBins = 1 << RB;
  constexpr int NW = NT / kWave;
  static_assert(kBins == 4 * NT, "four digit bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  *reinterpret_cast<uint4*>(hbin2 + 4 * tid) = make_uint4(0u, 0u, 0u, 0u);   // round 0's histogram
  uint64_t mn = ~0ull, mx = 0ull;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    if (v[u] != 0ull) {
      mn = v[u] < mn ? v[u] : mn;
      mx = v[u] > mx ? v[u] : mx;
    }
  }
  for (uint32_t f = tid; f < next; f += NT) {
    const uint64_t x = ext[f];
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  block_minmax_u64<NT>(mn, mx, tmp);                         // (its barriers order the clear)
  const uint64_t diff = mn ^ mx;
  int hi = diff ? 64 - __clzll((long long)diff) : 0;         // bits [hi-1 : 0] still open
  uint64_t prefix = hi == 64 ? 0ull : (mx >> hi) << hi;
  int buf = 0;
  while (true) {
    uint32_t* hb = hbin2 + buf * kBins;
    const int wd = hi < RB ? hi : RB;
    const int sh = hi - wd;
    const uint32_t dmask = (1u << wd) - 1u;
#pragma unroll
    for (int u = 0; u < SPT; ++u)
      if (v[u] != 0ull && (hi == 64 || (v[u] >> hi) == (prefix >> hi)))
        atomicAdd(&hb[(uint32_t)(v[u] >> sh) & dmask], 1u);
    for (uint32_t f = tid; f < next; f += NT) {
      const uint64_t x = ext[f];
      if (hi == 64 || (x >> hi) == (prefix >> hi)) atomicAdd(&hb[(uint32_t)(x >> sh) & dmask], 1u);
    }
    __syncthreads();
    // thread t holds digits kBins-1-4t .. kBins-4-4t (descending; digits >= 2^wd are empty)
    const uint4 x = *reinterpret_cast<const uint4*>(hb + kBins - 4 - 4 * tid);
    *reinterpret_cast<uint4*>(hbin2 + (buf ^ 1) * kBins + 4 * tid) = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t hv[4] = {x.w, x.z, x.y, x.x};
    const uint32_t tsum = hv[0] + hv[1] + hv[2] + hv[3];
    const uint32_t incl = wave_incl_scan(tsum);
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    uint32_t ex = incl - tsum;
#pragma unroll
    for (int w = 0; w < NW; ++w) ex += w < wave ? tmp[w] : 0u;
    if (ex < need && need <= ex + tsum) {
      uint32_t acc = ex;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc < need && need <= acc + hv[i]) {
          misc[0] = (uint32_t)(kBins - 1 - (4 * tid + i));
          misc[1] = acc;
          misc[2] = hv[i];
        }
        acc += hv[i];
      }
    }
    __syncthreads();
    need -= misc[1];
    prefix |= (uint64_t)misc[0] << sh;
    const bool done = misc[2] == need || sh == 0;
    hi = sh;
    buf ^= 1;
    if (done) break;
  }
  return prefix;
}

template <int FT>
__global__ __launch_bounds__(FT) void select_local_kernel(
    const float* __restrict__ scores, const uint64_t* __restrict__ cand_g, const uint4* __restrict__ meta_g,
    const int32_t* __restrict__ q_pos, int64_t N, int64_t sstride, int m, int k, int nch, int klocal, int64_t chunk,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int NT = FT;
  constexpr int SPT = kLocalCap / NT;                         // staged slots per thread
  __shared__ uint64_t cand_l[kExpCap];                       // candidates added by expansion
  __shared__ uint32_t bits_l[kLdsBitmapKeys / 32];           // also kth_largest's histogram
  __shared__ __attribute__((aligned(16))) uint32_t hbin_l[2 << kLocalRadixBits];   // kth_largest_regs' histograms
  __shared__ uint32_t mcnt[kMaxLocalChunks];
  __shared__ uint32_t mnv[kMaxLocalChunks];
  __shared__ uint64_t mfloor[kMaxLocalChunks];
  __shared__ uint32_t tmp[4 * NT / kWave];
  __shared__ uint32_t misc[8];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t n = vis_blocks(q_pos, row, m, N);
  const uint32_t kk = (uint32_t)k < n ? (uint32_t)k : n;
  int32_t* orow = out_idx + row * k;
  float* srow = out_score ? out_score + row * k : nullptr;
  const float* sc = scores + row * sstride;
  if (kk == 0) {
    for (int p = tid; p < k; p += NT) {
      orow[p] = -1;
      if (srow) srow[p] = -INFINITY;
    }
    return;
  }
  // 1. the chunks' lists and their counts in one load round; slots past a chunk's count
  //    become 0 (below every real composite).  Counts are clamped to what the index
  //    workgroups can have written.
  const uint32_t nslot = (uint32_t)nch * (uint32_t)klocal;
  const uint64_t* cg = cand_g + row * (int64_t)nslot;
  uint64_t v[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const uint32_t f = tid + u * NT;
    v[u] = f < nslot ? cg[f] : 0ull;
  }
  for (int c = tid; c < nch; c += NT) {
    const uint4 mm = meta_g[row * nch + c];
    const int64_t keys = N - (int64_t)c * chunk < chunk ? N - (int64_t)c * chunk : chunk;
    DSV4_DCHECK((int64_t)mm.y <= keys && mm.x <= (uint32_t)klocal && mm.x <= mm.y, kDbgLocalMeta);
    const uint32_t nvc = (int64_t)mm.y < keys ? mm.y : (uint32_t)keys;
    const uint32_t kept = mm.x < (uint32_t)klocal ? mm.x : (uint32_t)klocal;
    mnv[c] = nvc;
    mcnt[c] = kept < nvc ? kept : nvc;
    mfloor[c] = ((uint64_t)mm.w << 32) | mm.z;
  }
  __syncthreads();
  uint32_t nval = 0;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const uint32_t f = tid + u * NT;
    const uint32_t c = f / (uint32_t)klocal;
    const bool ok = f < nslot && f - c * (uint32_t)klocal < mcnt[c < (uint32_t)nch ? c : 0];
    v[u] = ok ? v[u] : 0ull;
    nval += ok ? 1u : 0u;
  }
  uint32_t valid;
  block_scan<NT>(nval, tmp, &valid);
  // 2. the threshold among the kept candidates (none if they are fewer than kk: then every
  //    chunk with omitted keys is expanded whole)
  uint64_t T = 0;
  if (valid >= kk) T = kth_largest_regs<NT, SPT, kLocalRadixBits>(v, cand_l, 0u, kk, hbin_l, tmp, misc);
  // 3. chunks that may hide keys above the threshold (checked in parallel; usually none)
  bool hidden = false;
  for (int c = tid; c < nch; c += NT) hidden |= mnv[c] > mcnt[c] && (valid < kk || mfloor[c] > T);
  const bool any_hidden = __syncthreads_or(hidden);
  bool fallback = false;
  uint32_t nexp = 0;
  if (any_hidden) {
    if (tid == 0) misc[4] = 0u;
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      if (!(mnv[c] > mcnt[c] && (valid < kk || mfloor[c] > T))) continue;
      const int64_t k0 = (int64_t)c * chunk;
      for (uint32_t i = tid; i < mnv[c]; i += NT) {
        const uint64_t x = comp_key(sc[k0 + i], (uint32_t)(k0 + i));
        if (x > T && x < mfloor[c]) {
          const uint32_t at = atomicAdd(&misc[4], 1u);
          if (at < (uint32_t)kExpCap) cand_l[at] = x;
        }
      }
    }
    __syncthreads();
    nexp = misc[4];
    fallback = nexp > (uint32_t)kExpCap;
    if (fallback) {   // rare: the whole row from the stored scores
      T = kth_largest<NT>([&](uint32_t f) -> uint64_t { return comp_key(sc[f], f); }, n, kk, bits_l, tmp, misc);
    } else {
      T = kth_largest_regs<NT, SPT, kLocalRadixBits>(v, cand_l, nexp, kk, hbin_l, tmp, misc);
    }
  }
  // 4. no chunk widened (the usual case): every chunk's list is in ascending key order and
  //    the chunks follow each other in slot order (slot f = u NT + tid), so the selected
  //    slots are compacted in slot order by one block scan of 16-bit counters, two slots
  //    per word
  if (!any_hidden) {
    constexpr int NW = NT / kWave;
    constexpr int NWD = (SPT + 1) / 2;
    static_assert(NW * NWD <= 4 * NT / kWave, "scan words fit in tmp");
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t cw[NWD], inc[NWD];
#pragma unroll
    for (int j = 0; j < NWD; ++j) {
      uint32_t f2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = 2 * j + h;
        if (u < SPT) {
          const uint32_t key = ~(uint32_t)v[u];
          DSV4_DCHECK(v[u] == 0ull || v[u] < T || key < n, kDbgCandIndex);
          f2 |= (v[u] != 0ull && v[u] >= T && key < n ? 1u : 0u) << (16 * h);
        }
      }
      cw[j] = f2;
      inc[j] = wave_incl_scan(f2);
      if (lane == 63) tmp[wave * NWD + j] = inc[j];
    }
    __syncthreads();
    uint32_t before[NWD], tot[NWD];
#pragma unroll
    for (int j = 0; j < NWD; ++j) before[j] = tot[j] = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
#pragma unroll
      for (int j = 0; j < NWD; ++j) {
        const uint32_t x = tmp[w * NWD + j];
        before[j] += w < wave ? x : 0u;
        tot[j] += x;
      }
    }
    uint32_t acc = 0;                                        // selected slots of earlier u
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const int j = u >> 1, sh = (u & 1) * 16;
      const uint32_t pos = acc + (((before[j] + inc[j] - cw[j]) >> sh) & 0xffffu);
      if (((cw[j] >> sh) & 1u) && pos < (uint32_t)k) {
        const uint32_t key = ~(uint32_t)v[u];
        orow[pos] = (int32_t)key;
        if (srow) srow[pos] = sc[key];
      }
      acc += (tot[j] >> sh) & 0xffffu;
    }
    for (int64_t p = (int64_t)acc + tid; p < k; p += NT) {
      orow[p] = -1;
      if (srow) srow[p] = -INFINITY;
    }
    return;
  }
  // 5. otherwise mark the selection in the bitmap
  const int64_t wn = ((int64_t)n + 31) / 32;
  for (int64_t w = tid; w < wn; w += NT) bits_l[w] = 0u;
  __syncthreads();
  if (!fallback) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const uint32_t j = ~(uint32_t)v[u];
      DSV4_DCHECK(v[u] == 0ull || v[u] < T || j < n, kDbgCandIndex);
      if (v[u] != 0ull && v[u] >= T && j < n) atomicOr(&bits_l[j >> 5], 1u << (j & 31));
    }
    for (uint32_t f = tid; f < nexp; f += NT) {
      const uint64_t x = cand_l[f];
      const uint32_t j = ~(uint32_t)x;
      DSV4_DCHECK(x < T || j < n, kDbgCandIndex);
      if (x >= T && j < n) atomicOr(&bits_l[j >> 5], 1u << (j & 31));
    }
  } else {
    for (uint32_t j = tid; j < n; j += NT)
      if (comp_key(sc[j], j) >= T) atomicOr(&bits_l[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // 6. compaction: thread t takes WPT consecutive words per round
  constexpr int WPT = (kLdsBitmapKeys / 32) / NT;
  uint32_t base_off = 0;
  for (int64_t r0 = 0; r0 < wn; r0 += WPT * NT) {
    const int64_t w0 = r0 + (int64_t)tid * WPT;
    uint32_t wv[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) wv[i] = w0 + i < wn ? bits_l[w0 + i] : 0u;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < WPT; ++i) cnt += __popc(wv[i]);
    uint32_t rtot;
    uint32_t off = base_off + block_scan<NT>(cnt, tmp, &rtot);
    for (int i = 0; i < WPT; ++i) {
      uint32_t b_ = wv[i];
      while (b_) {
        const int bpos = __ffs(b_) - 1;
        b_ &= b_ - 1;
        const int64_t j = (w0 + i) * 32 + bpos;
        if (off < (uint32_t)k) {
          orow[off] = (int32_t)j;
          if (srow) srow[off] = sc[j];
        }
        ++off;
      }
    }
    base_off += rtot;
  }
  for (int64_t p = (int64_t)base_off + tid; p < k; p += NT) {
    orow[p] = -1;
    if (srow) srow[p] = -INFINITY;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Launch plan of one csa_index_topk call, shared by the workspace query and the launch.
struct TopkPlan {
  bool local = false;      // local candidates + one finish pass (else histogram, scan, finish)
  int qtw = 1;             // query tiles per index workgroup
  int64_t chunk = 0;       // keys per index workgroup (MFMA kernels)
  int64_t nch = 0;         // index workgroups (key chunks) per query group
  int klocal = 0;          // candidates a chunk keeps (local path)
  size_t scores = 0, hist = 0, bitmap = 0, cand = 0, ccount = 0, thr = 0, cloc = 0, meta = 0, total = 0;
};

inline int64_t tiles_per_step_host(int kind, int DI) {
  return kind == KEY_BF16 ? (DI >= 256 ? 2 : 4) : (kind == KEY_FP8 && DI >= 256 ? 4 : 8);
}

TopkPlan plan_topk(const IndexArgs& a) {
  TopkPlan p;
  const int64_t R = a.B * a.Q, N = a.N;
  if (a.kind != KEY_F32 && N > 0) {
    const int64_t QPT = 16 / a.HI;
    // many queries per sequence (a prefill chunk): 4 query tiles (8 queries of one sequence)
    // per workgroup at the common indexer shape, so that every key tile feeds 4 MFMA row
    // blocks; a decode call (few queries per sequence, any batch) keeps one query tile and
    // streams its keys once
    p.qtw = (a.DI == 128 && a.HI == 8 && a.Q >= 8 && R >= 64) ? 4 : 1;
    const int64_t nw = (p.qtw > 1 && !a.pool.on) ? 8 : 4;   // waves per index workgroup
    const int64_t tpw = p.qtw == 1 ? tiles_per_step_host(a.kind, a.DI) : (a.kind == KEY_FP8 && nw == 4 ? 4 : 2);
    const int64_t KPS = tpw * 16 * nw;
    const int64_t QT = (a.Q + QPT - 1) / QPT, QG = (QT + p.qtw - 1) / p.qtw;
    int64_t chunk;
    if (p.qtw > 1) {                     // at least about 1024 workgroups over the whole call
      int64_t chunks = 1024 / (a.B * QG);
      if (chunks < 1) chunks = 1;
      // a multiple of the 8 XCDs: workgroup i runs on XCD i % 8, so with the key ranges as
      // the grid's fastest dimension each XCD reads one range of every sequence and its L2
      // keeps that range for all the query groups (one 66K-key prefill row: 1 MB of fp8
      // keys per XCD, against 4 MB per range with three ranges)
      chunks = (chunks + kXcds - 1) / kXcds * kXcds;
      chunk = (N + chunks - 1) / chunks;
    } else {                             // about two workgroups per CU over the whole call
      chunk = (N * (a.B * QT) + 511) / 512;
    }
    if (chunk > kMaxIndexChunk) chunk = kMaxIndexChunk;    // 16-bit LDS bin counters
    chunk = ((chunk + KPS - 1) / KPS) * KPS;
    if (chunk < KPS) chunk = KPS;
    if (p.qtw == 1 && N <= kLdsBitmapKeys) {
      const int64_t lc = chunk < kLocalChunk ? chunk : kLocalChunk;   // both multiples of KPS
      const int64_t nch = (N + lc - 1) / lc;
      if (nch <= kMaxLocalChunks) {
        int64_t kl = kLocalCap / nch;
        if (kl > kLocalKeep) kl = kLocalKeep;
        if (kl > a.k) kl = a.k;
        p.local = true;
        chunk = lc;
        p.klocal = (int)kl;
      }
    }
    p.chunk = chunk;
    p.nch = (N + chunk - 1) / chunk;
  }
  // workspace regions
  const int64_t sstride = ((N + 63) / 64) * 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.scores = take((size_t)R * sstride * 4);
  if (p.local) {
    p.cloc = take((size_t)R * p.nch * p.klocal * 8);
    p.meta = take((size_t)R * p.nch * 16);
  } else {
    const int64_t words = ((N + 127) / 128) * 4;             // bitmap rows of 16-byte multiples
    p.hist = take((size_t)R * kHistBins * 4);
    p.bitmap = take((size_t)R * words * 4);
    p.cand = take((size_t)R * N * 8);
    p.ccount = take((size_t)R * ((N + kScanKeys - 1) / kScanKeys) * 4);
    p.thr = take((size_t)R * 2 * 4);
  }
  p.total = off;
  return p;
}

struct IndexBufs {
  float* scores;
  uint32_t* hist;
  uint64_t* cloc;
  uint4* meta;
};

template <int KIND, int DI, int HI, int QTW, bool kLocal, int NW = 4>
hipError_t launch_mfma_q(const IndexArgs& a, const TopkPlan& p, const IndexBufs& w, hipStream_t st) {
  constexpr int QPT = 16 / HI;
  const int64_t QT = (a.Q + QPT - 1) / QPT;
  const int64_t QG = (QT + QTW - 1) / QTW;
  // the kernel clears and uses QPT histogram slots for each of its non-empty query tiles
  // (kLocal: one per query of its tile); the local selection adds the chunk's scores of
  // each query and its own scratch
  const int64_t tiles = QTW < QT ? QTW : QT;
  // pooling of the newest block (csa_pool_index_topk): the K|V rows' job on extra grid rows
  PoolDev pd{};
  int kv_rows = 0;
  if (a.pool.on) {
    pd.on = 1;
    pd.index_rows = (int)(a.B * QG);
    pd.kv_fp8 = a.pool.y_dt == 4;
    pd.m = a.m;
    pd.nblk = a.B;
    pd.x2 = reinterpret_cast<const uint16_t*>(a.pool.x2);
    pd.x2_bs = a.pool.x2_bs * DI;
    pd.gate = a.pool.gate;
    pd.bias = a.pool.bias;
    pd.row = a.pool.row;
    pd.lpr2 = DI / 8;                                          // bf16: 8 channels per lane
    pd.spb2 = 1;                                               // a power of two, lpr2 * spb2 <= 64
    while (2 * pd.spb2 <= a.m && 2 * pd.spb2 * pd.lpr2 <= kWave) pd.spb2 *= 2;
    CompressArgs ca;
    ca.x = a.pool.x; ca.x_f32 = false; ca.gate = a.pool.gate; ca.bias = a.pool.bias;
    ca.B = a.B; ca.T = a.m; ca.C = a.pool.C; ca.m = a.m;
    ca.x_bs = a.pool.x_bs; ca.y_bs = a.pool.y_bs; ca.y = a.pool.y; ca.y_scale = a.pool.y_scale; ca.y_dt = a.pool.y_dt;
    pd.kv = a.pool.y_dt == 4 ? pool::make_job_packed<uint16_t, 4>(ca) : pool::make_job_packed<uint16_t, 1>(ca);
    kv_rows = (int)((pd.kv.grid + p.nch - 1) / p.nch);
  }
  dim3 grid((unsigned)p.nch, (unsigned)(a.B * QG + kv_rows));
  size_t smem = (size_t)(kLocal ? (a.Q < QPT ? a.Q : QPT) : tiles * QPT) * kHistWords * sizeof(uint32_t);
  if (kLocal)
    smem += (size_t)(a.Q < QPT ? a.Q : QPT) * p.chunk * sizeof(float) +
            (size_t)((1 << kRadixBits) + 2 * NW + 8) * sizeof(uint32_t);
  if (a.pool.on) {                                           // a pooling workgroup's states
    const size_t part = (size_t)pool::kThreads * (pool::XVec<uint16_t>::N + 2) * sizeof(float);
    smem = smem > part ? smem : part;
  }
  // at most two decode workgroups per CU: with three the dispatcher fills some CUs before
  // others, and at the per-CU read rate the fullest CUs set the kernel's end (measured:
  // 37.5 us instead of 34.8 us for the 1M-context decode call)
  if (kLocal && smem < kMinLocalLds) smem = kMinLocalLds;
  const int64_t sstride = ((a.N + 63) / 64) * 64;
  // one query group per sequence: every key is read by one workgroup of the call, so the
  // keys are streamed with the non-temporal hint; with several groups the caches serve the
  // repeated reads (multi-query calls always run with QTW > 1 or several groups)
  auto go = [&](auto kern) {
    if (smem > 65536) hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    DSV4_LAUNCH_MAIN(kern, grid, dim3(NW * kWave), smem, st, reinterpret_cast<const uint8_t*>(a.qi), a.qi_scale, a.wi,
                     reinterpret_cast<const uint8_t*>(a.ki), a.ki_scale, a.q_pos, a.N, a.k_bs, a.Q, a.m, p.chunk,
                     w.scores, sstride, w.hist, w.cloc, w.meta, p.klocal, (int)p.nch, pd);
  };
  if constexpr (NW == 4) {
    if (QTW == 1 && QG == 1) go(index_mfma_kernel<KIND, DI, HI, QTW, (QTW == 1), kLocal>);
    else go(index_mfma_kernel<KIND, DI, HI, QTW, false, kLocal>);
  } else {
    if (QTW == 1 && QG == 1) go(index_mfma_kernel<KIND, DI, HI, QTW, (QTW == 1), kLocal, NW>);
    else go(index_mfma_kernel<KIND, DI, HI, QTW, false, kLocal, NW>);
  }
  return hipGetLastError();
}

template <int KIND, int DI>
hipError_t launch_mfma_di(const IndexArgs& a, const TopkPlan& p, const IndexBufs& w, hipStream_t st) {
  if constexpr (DI == 128) {
    // many queries: eight waves per workgroup (two workgroups and 16 waves per CU with the
    // same 64 KB of histograms), four when the call also pools a block (its pooling body
    // runs on 256 threads)
    if (p.qtw == 4) return a.pool.on ? launch_mfma_q<KIND, DI, 8, 4, false>(a, p, w, st)
                                     : launch_mfma_q<KIND, DI, 8, 4, false, 8>(a, p, w, st);
  }
  if (p.local) {
    switch (a.HI) {
      case 4: return launch_mfma_q<KIND, DI, 4, 1, true, kLocalWaves>(a, p, w, st);
      case 8: return launch_mfma_q<KIND, DI, 8, 1, true, kLocalWaves>(a, p, w, st);
      default: return launch_mfma_q<KIND, DI, 16, 1, true, kLocalWaves>(a, p, w, st);
    }
  }
  switch (a.HI) {
    case 4: return launch_mfma_q<KIND, DI, 4, 1, false>(a, p, w, st);
    case 8: return launch_mfma_q<KIND, DI, 8, 1, false>(a, p, w, st);
    default: return launch_mfma_q<KIND, DI, 16, 1, false>(a, p, w, st);
  }
}

template <int KIND>
hipError_t launch_mfma(const IndexArgs& a, const TopkPlan& p, const IndexBufs& w, hipStream_t st) {
  if constexpr (KIND == KEY_MXFP4_Q4) {    // 128-deep FP4 MFMA steps: DI of 128 or 256
    if (a.DI == 128) return launch_mfma_di<KIND, 128>(a, p, w, st);
    return launch_mfma_di<KIND, 256>(a, p, w, st);
  }
  switch (a.DI) {
    case 32: return launch_mfma_di<KIND, 32>(a, p, w, st);
    case 64: return launch_mfma_di<KIND, 64>(a, p, w, st);
    case 128: return launch_mfma_di<KIND, 128>(a, p, w, st);
    default: return launch_mfma_di<KIND, 256>(a, p, w, st);
  }
}

}  // namespace

size_t topk_workspace_bytes(const IndexArgs& a) { return a.B * a.Q > 0 ? plan_topk(a).total : 0; }

hipError_t launch_index_topk(const IndexArgs& a, void* ws, hipStream_t st) {
  const int64_t R = a.B * a.Q;
  if (R == 0) return hipSuccess;
  const TopkPlan p = plan_topk(a);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  IndexBufs w;
  w.scores = reinterpret_cast<float*>(base + p.scores);
  w.hist = p.local ? nullptr : reinterpret_cast<uint32_t*>(base + p.hist);
  w.cloc = p.local ? reinterpret_cast<uint64_t*>(base + p.cloc) : nullptr;
  w.meta = p.local ? reinterpret_cast<uint4*>(base + p.meta) : nullptr;
  const int64_t sstride = ((a.N + 63) / 64) * 64;
  hipError_t e;
  if (p.local) {
    // pass 1: scores, each chunk's local candidates; pass 2: one workgroup per row
    if (a.kind == KEY_BF16) e = launch_mfma<KEY_BF16>(a, p, w, st);
    else if (a.kind == KEY_FP8) e = launch_mfma<KEY_FP8>(a, p, w, st);
    else if (a.kind == KEY_MXFP4_Q4) e = launch_mfma<KEY_MXFP4_Q4>(a, p, w, st);
    else e = launch_mfma<KEY_MXFP4>(a, p, w, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_local_kernel<kLocalFinThreads>, dim3((unsigned)R), dim3(kLocalFinThreads), 0, st,
                       w.scores, w.cloc, w.meta, a.q_pos, a.N, sstride, a.m, a.k, (int)p.nch, p.klocal, p.chunk,
                       a.out_idx, a.out_score);
    return hipGetLastError();
  }
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + p.bitmap);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + p.cand);
  uint32_t* ccount = reinterpret_cast<uint32_t*>(base + p.ccount);
  uint32_t* thr = reinterpret_cast<uint32_t*>(base + p.thr);
  const int64_t nclear = R * kHistBins;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclear + 1023) / 1024 < 256 ? (nclear + 1023) / 1024 : 256)),
                     dim3(1024), 0, st, w.hist, nclear);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N > 0) {
    if (a.kind == KEY_F32) {
      dim3 grid((unsigned)((a.N + kThreads - 1) / kThreads), (unsigned)R);
      size_t smem = (kHistWords + (size_t)a.HI * a.DI + a.HI) * 4;
      DSV4_LAUNCH_MAIN(index_f32_kernel, grid, dim3(kThreads), smem, st, reinterpret_cast<const float*>(a.qi),
                       a.wi, reinterpret_cast<const float*>(a.ki), a.q_pos, a.N, a.k_bs, a.Q, a.HI, a.DI, a.m,
                       w.scores, sstride, w.hist);
      e = hipGetLastError();
    } else if (a.kind == KEY_BF16) e = launch_mfma<KEY_BF16>(a, p, w, st);
    else if (a.kind == KEY_FP8) e = launch_mfma<KEY_FP8>(a, p, w, st);
    else if (a.kind == KEY_MXFP4_Q4) e = launch_mfma<KEY_MXFP4_Q4>(a, p, w, st);
    else e = launch_mfma<KEY_MXFP4>(a, p, w, st);
    if (e != hipSuccess) return e;
  }
  // selection: pass 1 over all rows x key ranges, pass 2 one workgroup per row
  if (a.N == 0) {
    hipLaunchKernelGGL(select_finish_kernel<kLdsBitmapKeysSmall>, dim3((unsigned)R), dim3(kFinThreads), 0, st,
                       w.scores, bitmap, cand, ccount, thr, a.q_pos, a.N, (int64_t)0, (int64_t)0, a.m, a.k, 0,
                       (int64_t)kScanKeys, a.out_idx, a.out_score);
    return hipGetLastError();
  }
  const int64_t words = ((a.N + 127) / 128) * 4;
  const int64_t rk = scan_keys(R);        // keys per range (the workspace holds counts for kScanKeys)
  const int64_t nrg = (a.N + rk - 1) / rk;
  hipLaunchKernelGGL(select_threshold_kernel, dim3((unsigned)R), dim3(kScanThreads), 0, st, w.hist, thr, a.q_pos, a.N,
                     a.m, a.k);
  if (rk == kScanKeysMany)
    hipLaunchKernelGGL(select_scan_kernel<kScanKeysMany>, dim3((unsigned)nrg, (unsigned)R), dim3(kScanThreads), 0, st,
                       w.scores, bitmap, cand, ccount, thr, a.q_pos, a.N, sstride, words, a.m, a.k);
  else
    hipLaunchKernelGGL(select_scan_kernel<kScanKeys>, dim3((unsigned)nrg, (unsigned)R), dim3(kScanThreads), 0, st,
                       w.scores, bitmap, cand, ccount, thr, a.q_pos, a.N, sstride, words, a.m, a.k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N <= kLdsBitmapKeysSmall)
    hipLaunchKernelGGL(select_finish_kernel<kLdsBitmapKeysSmall>, dim3((unsigned)R), dim3(kFinThreads), 0, st,
                       w.scores, bitmap, cand, ccount, thr, a.q_pos, a.N, sstride, words, a.m, a.k, (int)nrg, rk,
                       a.out_idx, a.out_score);
  else if (a.N <= kLdsBitmapKeys)
    hipLaunchKernelGGL(select_finish_kernel<kLdsBitmapKeys>, dim3((unsigned)R), dim3(kFinThreads), 0, st, w.scores,
                       bitmap, cand, ccount, thr, a.q_pos, a.N, sstride, words, a.m, a.k, (int)nrg, rk, a.out_idx,
                       a.out_score);
  else
    hipLaunchKernelGGL(select_finish_kernel<0>, dim3((unsigned)R), dim3(kFinThreads), 0, st, w.scores, bitmap,
                       cand, ccount, thr, a.q_pos, a.N, sstride, words, a.m, a.k, (int)nrg, rk, a.out_idx,
                       a.out_score);
  return hipGetLastError();
}

DSV4_DEBUG_READER(debug_flags_index)

}  // namespace dsv4
