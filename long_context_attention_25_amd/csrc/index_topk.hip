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
//      (16 rows = QPT queries x HI heads, 16 keys per tile, K = 32 per step; fp8 keys
//      with DI >= 128 and MXFP4 queries: the scaled MFMA, K = 128 per step).  The
//      epilogue applies ReLU, the head weights and the head sum, writes the fp32
//      scores and adds the top 12 bits of each score's order-preserving key into a
//      per-row histogram (LDS histogram, then one global atomic per non-empty bin).
//   2. select kernel, one workgroup per row: finds the threshold bin of the row from the
//      histogram, reads the row's scores once, marks the keys above the bin in an LDS
//      bitmap and collects the keys inside the bin as candidates, radix-selects the
//      remaining candidates by (score, lower index first), and compacts the bitmap into
//      ascending indices.
// The result is exact on the fp32 scores and independent of scheduling.
#include "common.hpp"
#include "launch.hpp"

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

// Writes one score and counts it in the LDS histogram of its query slot.
__device__ __forceinline__ void emit_score(float* scores, uint32_t* hist_l, int64_t row, int64_t sstride,
                                           int64_t N, int64_t key, uint32_t nvis, float v) {
  if (key >= N) return;
  bool vis = key < (int64_t)nvis;
  scores[row * sstride + key] = vis ? v : -INFINITY;
  if (vis) {
    const uint32_t bin = score_key(v) >> (32 - kHistBits);
    atomicAdd(&hist_l[bin >> 1], 1u << ((bin & 1u) << 4));
  }
}

__device__ __forceinline__ void flush_hist(const uint32_t* hist_l, uint32_t* hist_g, int64_t row) {
  for (int w = threadIdx.x; w < kHistWords; w += kThreads) {
    const uint32_t c = hist_l[w];
    if (c & 0xffffu) atomicAdd(&hist_g[row * kHistBins + 2 * w], c & 0xffffu);
    if (c >> 16) atomicAdd(&hist_g[row * kHistBins + 2 * w + 1], c >> 16);
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

// QTW query tiles (QTW * 16/HI queries) per workgroup: every key tile loaded is used by
// all of them (QTW > 1 when there are many queries, e.g. a prefill chunk).
template <int KIND, int DI, int HI, int QTW, bool kNT>
__global__ __launch_bounds__(kThreads) void index_mfma_kernel(
    const uint8_t* __restrict__ qi, const uint8_t* __restrict__ qsc, const float* __restrict__ wi,
    const uint8_t* __restrict__ ki, const uint8_t* __restrict__ ksc, const int32_t* __restrict__ q_pos, int64_t N,
    int64_t k_bs, int64_t Q, int m, int64_t chunk, float* __restrict__ scores, int64_t sstride,
    uint32_t* __restrict__ hist_g) {
  constexpr int QPT = 16 / HI;          // queries per 16-row MFMA tile
  constexpr int KS = DI / 32;
  constexpr int GPQ = HI / 4;           // lane groups per query slot
  extern __shared__ uint32_t hist_l[];  // [QTW * QPT][kHistWords]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
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
  constexpr int TPW = QTW == 1 ? tiles_per_step<KIND, DI>() : (KIND == KEY_FP8 ? 4 : 2);
  constexpr int KPS = TPW * 16 * 4;
  constexpr int E = GPQ < TPW ? GPQ : TPW;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  int64_t c1 = c0 + chunk;
  if (c1 > N) c1 = N;
  const int64_t klast = c1 - 1;
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
    nslots += nq[t] > 0 ? QPT : 0;
  }
  for (int i = threadIdx.x; i < nslots * kHistWords; i += kThreads) hist_l[i] = 0u;

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
  // last key, so loads never branch; only the score write is guarded.
  for (; base < c1; base += KPS) {
    const int64_t nb = base + KPS;
    if (nb < c1) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int64_t key = nb + u * 16 + col;
        nxt[u].template load<kNT>(kbase, sbase, key < klast ? key : klast, g, true);
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
              const auto& kt = cur[u + j];
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
              const auto& kt = cur[u + j];
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
                acc = mfma_fp8(__builtin_bit_cast(long, qa8[t][c]), cur[u + j].op(c), acc);
              else acc = mfma_bf16(bit_cast_to<bf16x8>(qa16[t][c]), cur[u + j].op(c), acc);
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
        if (owner[t] && key < c1)
          emit_score(scores, hist_l + (t * QPT + qs_c) * kHistWords, row_c[t], sstride, N, key, nvis[t], vs);
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) cur[u] = nxt[u];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < QTW; ++t)
    for (int s = 0; s < nq[t]; ++s)
      flush_hist(hist_l + (t * QPT + s) * kHistWords, hist_g, b * Q + (qt0 + t) * QPT + s);
}

// ------------------------------------------------------------------ selection
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
constexpr int kCandCap = 4096;                               // candidates staged in LDS by pass 2
constexpr int kRadixBits = 12;                               // digit width of pass 2's radix select

template <int KEYS>
__global__ __launch_bounds__(kScanThreads) void select_scan_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist_g, uint32_t* __restrict__ bitmap_g,
    uint64_t* __restrict__ cand_g, uint32_t* __restrict__ ccount, uint32_t* __restrict__ thr,
    const int32_t* __restrict__ q_pos, int64_t N, int64_t sstride, int64_t words, int m, int k) {
  __shared__ uint32_t tmp[kScanThreads / kWave];
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
  // issue the score loads first; the threshold is computed while they are in flight
  const float* sc = scores + row * sstride + c0;
  const int64_t c1 = (c0 + KEYS < (int64_t)n ? c0 + KEYS : (int64_t)n) - c0;   // keys in range
  constexpr int IT = KEYS / (4 * kScanThreads);
  float4 v[IT];
#pragma unroll
  for (int u = 0; u < IT; ++u) {
    const int64_t kb = (int64_t)(u * kScanThreads + tid) * 4;
    v[u] = kb < c1 ? reinterpret_cast<const float4*>(sc)[u * kScanThreads + tid]
                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  if (tid == 0) misc[2] = 0u;
  threshold_bin<kScanThreads>(hist_g + row * kHistBins, kk, tmp, misc);
  const uint32_t tbin = misc[0];
  if (blockIdx.x == 0 && tid == 0) {       // recorded once per row for pass 2
    thr[row * 2] = tbin;
    thr[row * 2 + 1] = misc[1];
  }

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
// kLdsBits: the row's bitmap is copied into LDS (N <= kLdsBitmapKeys).
template <bool kLdsBits>
__global__ __launch_bounds__(kFinThreads) void select_finish_kernel(
    const float* __restrict__ scores, uint32_t* __restrict__ bitmap_g, const uint64_t* __restrict__ cand_g,
    const uint32_t* __restrict__ ccount, const uint32_t* __restrict__ thr, const int32_t* __restrict__ q_pos,
    int64_t N, int64_t sstride, int64_t words, int m, int k, int nch, int64_t rkeys, int32_t* __restrict__ out_idx,
    float* __restrict__ out_score) {
  constexpr int NT = kFinThreads;
  constexpr int kBins = 1 << kRadixBits;
  constexpr int BPT = kBins / NT;
  static_assert(BPT >= 1 && kBins % NT == 0, "digit bins per thread");
  __shared__ uint32_t bits_l[kLdsBits ? kLdsBitmapKeys / 32 : 1];
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
    return c_ < (uint64_t)keys ? c_ : (uint32_t)keys;
  };
  uint2 th = *reinterpret_cast<const uint2*>(thr + row * 2);
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

template <int KIND, int DI, int HI, int QTW>
hipError_t launch_mfma_q(const IndexArgs& a, float* scores, uint32_t* hist, int64_t chunk, hipStream_t st) {
  constexpr int QPT = 16 / HI;
  constexpr int KPS = (QTW == 1 ? tiles_per_step<KIND, DI>() : (KIND == KEY_FP8 ? 4 : 2)) * 16 * 4;
  const int64_t QT = (a.Q + QPT - 1) / QPT;
  const int64_t QG = (QT + QTW - 1) / QTW;
  if (QTW > 1) {                          // about 1024 workgroups over the whole call
    int64_t chunks = 1024 / (a.B * QG);
    if (chunks < 1) chunks = 1;
    chunk = (a.N + chunks - 1) / chunks;
  }
  if (chunk > kMaxIndexChunk) chunk = kMaxIndexChunk;    // 16-bit LDS bin counters
  chunk = ((chunk + KPS - 1) / KPS) * KPS;
  if (chunk < KPS) chunk = KPS;
  dim3 grid((unsigned)((a.N + chunk - 1) / chunk), (unsigned)(a.B * QG));
  // the kernel clears and uses QPT histogram slots for each of its non-empty query tiles
  const int64_t tiles = QTW < QT ? QTW : QT;
  const size_t smem = (size_t)(tiles * QPT) * kHistWords * sizeof(uint32_t);
  // one query group per sequence: every key is read by one workgroup of the call, so the
  // keys are streamed with the non-temporal hint; with several groups the caches serve the
  // repeated reads (multi-query calls always run with QTW > 1 or several groups)
  if (QTW == 1 && QG == 1)
    DSV4_LAUNCH_MAIN((index_mfma_kernel<KIND, DI, HI, QTW, (QTW == 1)>), grid, dim3(kThreads), smem, st,
                     reinterpret_cast<const uint8_t*>(a.qi), a.qi_scale, a.wi, reinterpret_cast<const uint8_t*>(a.ki),
                     a.ki_scale, a.q_pos, a.N, a.k_bs, a.Q, a.m, chunk, scores, ((a.N + 63) / 64) * 64, hist);
  else
    DSV4_LAUNCH_MAIN((index_mfma_kernel<KIND, DI, HI, QTW, false>), grid, dim3(kThreads), smem, st,
                     reinterpret_cast<const uint8_t*>(a.qi), a.qi_scale, a.wi, reinterpret_cast<const uint8_t*>(a.ki),
                     a.ki_scale, a.q_pos, a.N, a.k_bs, a.Q, a.m, chunk, scores, ((a.N + 63) / 64) * 64, hist);
  return hipGetLastError();
}

template <int KIND, int DI>
hipError_t launch_mfma_di(const IndexArgs& a, float* scores, uint32_t* hist, int64_t chunk, hipStream_t st) {
  // many queries per sequence (a prefill chunk): 4 query tiles (8 queries of one sequence)
  // per workgroup at the common indexer shape, so that every key tile feeds 4 MFMA row
  // blocks; a decode call (few queries per sequence, any batch) keeps one query tile and
  // streams its keys once
  if constexpr (DI == 128) {
    if (a.HI == 8 && a.Q >= 8 && a.B * a.Q >= 64) return launch_mfma_q<KIND, DI, 8, 4>(a, scores, hist, chunk, st);
  }
  switch (a.HI) {
    case 4: return launch_mfma_q<KIND, DI, 4, 1>(a, scores, hist, chunk, st);
    case 8: return launch_mfma_q<KIND, DI, 8, 1>(a, scores, hist, chunk, st);
    default: return launch_mfma_q<KIND, DI, 16, 1>(a, scores, hist, chunk, st);
  }
}

template <int KIND>
hipError_t launch_mfma(const IndexArgs& a, float* scores, uint32_t* hist, int64_t chunk, hipStream_t st) {
  if constexpr (KIND == KEY_MXFP4_Q4) {    // 128-deep FP4 MFMA steps: DI of 128 or 256
    if (a.DI == 128) return launch_mfma_di<KIND, 128>(a, scores, hist, chunk, st);
    return launch_mfma_di<KIND, 256>(a, scores, hist, chunk, st);
  }
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
  const int64_t nch = (N + kScanKeys - 1) / kScanKeys;
  return align256((size_t)R * sstride * 4) + align256((size_t)R * kHistBins * 4) + align256((size_t)R * words * 4) +
         align256((size_t)R * N * 8) + align256((size_t)R * nch * 4) + align256((size_t)R * 2 * 4);
}

TopkWorkspace topk_workspace_carve(void* base, int64_t R, int64_t N) {
  int64_t words = ((N + 127) / 128) * 4;   // rows of 16-byte multiples
  uint8_t* p = reinterpret_cast<uint8_t*>(base);
  TopkWorkspace w;
  w.scores = reinterpret_cast<float*>(p);
  p += align256((size_t)R * (((N + 63) / 64) * 64) * 4);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * kHistBins * 4);
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * words * 4);
  w.cand = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)R * N * 8);
  w.ccount = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)R * ((N + kScanKeys - 1) / kScanKeys) * 4);
  w.thr = reinterpret_cast<uint32_t*>(p);
  return w;
}

hipError_t launch_index_topk(const IndexArgs& a, const TopkWorkspace& ws, hipStream_t st) {
  const int64_t R = a.B * a.Q;
  if (R == 0) return hipSuccess;
  const int64_t nclear = R * kHistBins;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)((nclear + 1023) / 1024 < 256 ? (nclear + 1023) / 1024 : 256)),
                     dim3(1024), 0, st, ws.hist, nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N > 0) {
    if (a.kind == KEY_F32) {
      dim3 grid((unsigned)((a.N + kThreads - 1) / kThreads), (unsigned)R);
      size_t smem = (kHistWords + (size_t)a.HI * a.DI + a.HI) * 4;
      DSV4_LAUNCH_MAIN(index_f32_kernel, grid, dim3(kThreads), smem, st, reinterpret_cast<const float*>(a.qi),
                         a.wi, reinterpret_cast<const float*>(a.ki), a.q_pos, a.N, a.k_bs, a.Q, a.HI, a.DI, a.m,
                         ws.scores, ((a.N + 63) / 64) * 64, ws.hist);
      e = hipGetLastError();
    } else {
      // about two workgroups per CU over the whole call
      int QPT = 16 / a.HI;
      int64_t rows = a.B * ((a.Q + QPT - 1) / QPT);
      int64_t per = (a.N * rows + 511) / 512;
      // (rounded to whole steps of the kernel inside launch_mfma_di)
      int64_t chunk = per;
      if (a.kind == KEY_BF16) e = launch_mfma<KEY_BF16>(a, ws.scores, ws.hist, chunk, st);
      else if (a.kind == KEY_FP8) e = launch_mfma<KEY_FP8>(a, ws.scores, ws.hist, chunk, st);
      else if (a.kind == KEY_MXFP4_Q4) e = launch_mfma<KEY_MXFP4_Q4>(a, ws.scores, ws.hist, chunk, st);
      else e = launch_mfma<KEY_MXFP4>(a, ws.scores, ws.hist, chunk, st);
    }
    if (e != hipSuccess) return e;
  }
  // selection: pass 1 over all rows x key ranges, pass 2 one workgroup per row
  if (a.N == 0) {
    hipLaunchKernelGGL(select_finish_kernel<true>, dim3((unsigned)R), dim3(kFinThreads), 0, st, ws.scores,
                       ws.bitmap, ws.cand, ws.ccount, ws.thr, a.q_pos, a.N, (int64_t)0, (int64_t)0, a.m, a.k, 0,
                       (int64_t)kScanKeys, a.out_idx, a.out_score);
    return hipGetLastError();
  }
  const int64_t words = ((a.N + 127) / 128) * 4;
  const int64_t sstride = ((a.N + 63) / 64) * 64;
  const int64_t rk = scan_keys(R);        // keys per range (the workspace holds counts for kScanKeys)
  const int64_t nch = (a.N + rk - 1) / rk;
  if (rk == kScanKeysMany)
    hipLaunchKernelGGL(select_scan_kernel<kScanKeysMany>, dim3((unsigned)nch, (unsigned)R), dim3(kScanThreads), 0, st,
                       ws.scores, ws.hist, ws.bitmap, ws.cand, ws.ccount, ws.thr, a.q_pos, a.N, sstride, words, a.m, a.k);
  else
    hipLaunchKernelGGL(select_scan_kernel<kScanKeys>, dim3((unsigned)nch, (unsigned)R), dim3(kScanThreads), 0, st,
                       ws.scores, ws.hist, ws.bitmap, ws.cand, ws.ccount, ws.thr, a.q_pos, a.N, sstride, words, a.m, a.k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.N <= kLdsBitmapKeys)
    hipLaunchKernelGGL(select_finish_kernel<true>, dim3((unsigned)R), dim3(kFinThreads), 0, st, ws.scores,
                       ws.bitmap, ws.cand, ws.ccount, ws.thr, a.q_pos, a.N, sstride, words, a.m, a.k, (int)nch, rk,
                       a.out_idx, a.out_score);
  else
    hipLaunchKernelGGL(select_finish_kernel<false>, dim3((unsigned)R), dim3(kFinThreads), 0, st, ws.scores,
                       ws.bitmap, ws.cand, ws.ccount, ws.thr, a.q_pos, a.N, sstride, words, a.m, a.k, (int)nch, rk,
                       a.out_idx, a.out_score);
  return hipGetLastError();
}

}  // namespace dsv4
