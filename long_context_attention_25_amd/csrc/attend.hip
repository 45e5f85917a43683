// CSA / HCA attention over compressed entries plus the sliding window, and the
// log-sum-exp merge, for gfx950.
//
// The key set of a query is the union of compressed entries (the top-k selected
// blocks for CSA, every visible block for HCA) and the raw window rows, attended as
// one softmax (honbul.tistory.com/221, "CSA: 압축한 뒤, 필요한 기억만 골라서 보기":
// compressed long-range memory and recent raw memory are used together; "HCA: 더
// 강하게 압축하고, 압축된 전체를 보기": every compressed entry, no selection;
// pogovet.com 상세 정리 §4).
//
// bf16 path (MQA, H <= 64 heads share one K/V):
//   grid = (key-range splits, B*Q); 4 waves, wave w owns heads 16w..16w+15.
//   Per 32-key sub-tile the K rows (gathered by index, or contiguous) are staged in
//   LDS as-is and the V rows are staged transposed (dims x keys, via byte
//   permutes of dword loads), while the next sub-tile's rows are already in flight
//   in registers.  S^T = K.Q^T comes from mfma_f32_16x16x32_bf16 with K as the
//   A operand, so each lane ends up holding 8 scores of ONE head; those scores,
//   exponentiated and rounded to bf16, are directly the B operand of
//   O^T += V^T.P^T with no data movement.  Online softmax in fp32 (exp2 with the
//   scale folded in).  Splits write fp32 partial (o, lse) that lse_merge combines.
// fp32 path: a plain VALU kernel, one workgroup per (query, head).
#include "common.hpp"
#include "launch.hpp"

namespace dsv4 {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;            // keys per sub-tile
constexpr int kTargetWorkgroups = 256;   // gfx950: 256 CUs, one attention workgroup each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct KeyRange {
  int64_t n_c;      // compressed part length (CSA: k list slots, HCA: visible blocks)
  int64_t r_lo;     // first window row
  int64_t n_tot;    // n_c + window rows
};

__device__ __forceinline__ KeyRange key_range(const AttendArgs& a, int64_t bq) {
  const int64_t b = bq / a.Q;
  const int64_t p = a.q_pos[bq];
  KeyRange r;
  if (a.csa) {
    r.n_c = a.k;
  } else {
    int64_t n = p < 0 ? 0 : (p + 1) / a.m;
    r.n_c = n < a.N ? n : a.N;
  }
  const int64_t wp0 = a.win_pos0[b];
  int64_t lo = p - a.W + 1 - wp0;
  int64_t hi = p + 1 - wp0;
  if (lo < 0) lo = 0;
  if (hi > a.L) hi = a.L;
  r.r_lo = lo;
  r.n_tot = r.n_c + (hi > lo ? hi - lo : 0);
  return r;
}

// Row (element offset into kc/vc or kw/vw) of list position `pos`; -1 if the slot is empty.
// Sets *win when the row comes from the window buffer.
__device__ __forceinline__ int64_t key_row(const AttendArgs& a, int64_t bq, const KeyRange& kr, int64_t pos,
                                           bool* win) {
  const int64_t b = bq / a.Q;
  *win = false;
  if (pos >= kr.n_tot) return -1;
  if (pos < kr.n_c) {
    int64_t j = a.csa ? (int64_t)a.idx[bq * a.k + pos] : pos;
    if (j < 0 || j >= a.N) return -1;
    return (b * a.kv_bs + j) * a.D;
  }
  *win = true;
  return (b * a.L + kr.r_lo + (pos - kr.n_c)) * a.D;
}

// ---------------------------------------------------------------------------- bf16 / MFMA
// Global row pointers (K and V) of list position `pos`; an empty slot points at a real
// row (compressed row 0, or window row 0 when there are no compressed rows) and is
// reported invalid, so tile loads never branch.
__device__ __forceinline__ bool key_ptrs(const AttendArgs& a, int64_t bq, const KeyRange& kr, int64_t pos,
                                         const uint16_t** kp, const uint16_t** vp) {
  const int64_t b = bq / a.Q;
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.kc) + b * a.kv_bs * a.D;
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.vc) + b * a.kv_bs * a.D;
  const uint16_t* kw = reinterpret_cast<const uint16_t*>(a.kw) + b * a.L * a.D;
  const uint16_t* vw = reinterpret_cast<const uint16_t*>(a.vw) + b * a.L * a.D;
  *kp = a.N > 0 ? kc : kw;
  *vp = a.N > 0 ? vc : vw;
  if (pos >= kr.n_tot) return false;
  if (pos < kr.n_c) {
    const int64_t j = a.csa ? (int64_t)a.idx[bq * a.k + pos] : pos;
    if (j < 0 || j >= a.N) return false;
    *kp = kc + j * a.D;
    *vp = vc + j * a.D;
    return true;
  }
  const int64_t r = kr.r_lo + (pos - kr.n_c);
  *kp = kw + r * a.D;
  *vp = vw + r * a.D;
  return true;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendArgs a, int64_t chunk, int splits,
                                                               float* __restrict__ o_part,
                                                               float* __restrict__ lse_part) {
  constexpr int KS = D / 32;               // MFMA k-steps over the head dim
  constexpr int KSTR = D + 8;              // LDS row stride of K (elements)
  constexpr int VSTR = kTile + 8;          // LDS row stride of V^T (elements)
  constexpr int KCH = D / 8;               // 16-byte chunks per row
  constexpr int KROWS = kThreads / KCH;    // K rows loaded per pass
  constexpr int KLD = kTile / KROWS;       // K loads (16 B) per thread and tile
  constexpr int DP = D / 2;                // dim pairs
  constexpr int KG = kThreads / DP;        // key groups for V
  constexpr int KPG = kTile / KG;          // V loads (4 B) per thread and tile, keys of one group
  constexpr int NREG = KLD * 4 > KPG ? KLD * 4 : KPG;
  constexpr int MC = 128;                  // keys per macro-chunk (softmax max taken over it)
  constexpr int TPM = MC / kTile;          // tiles per macro-chunk
  constexpr int LDS_ELEMS = (kTile * KSTR > D * VSTR) ? kTile * KSTR : D * VSTR;
  static_assert(KPG % 8 == 0, "V transpose needs groups of 8 keys");

  __shared__ __attribute__((aligned(16))) uint16_t tile[LDS_ELEMS];   // K rows or V^T, in turn
  __shared__ const uint16_t* kptr[2][MC];
  __shared__ const uint16_t* vptr[2][MC];
  __shared__ uint32_t valid[2][MC / 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t bq = blockIdx.y;
  const int split = blockIdx.x;
  const KeyRange kr = key_range(a, bq);
  const int64_t s0 = (int64_t)split * chunk;
  int64_t s1 = s0 + chunk;
  if (s1 > kr.n_tot) s1 = kr.n_tot;
  const int nmacro = s1 > s0 ? (int)((s1 - s0 + MC - 1) / MC) : 0;

  const int head = wave * 16 + col;
  const bool wave_on = wave * 16 < a.H;

  uint4 qop[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (bq * a.H + (wave_on ? head : 0)) * D + g * (D / 4);
#pragma unroll
    for (int c = 0; c < KS; ++c) qop[c] = wave_on ? gload_u4(qp + 8 * c) : make_uint4(0, 0, 0, 0);
  }
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  uint32_t reg[NREG];                      // the next tile in flight (K chunks or V dwords)
  const int kcol = (tid % KCH) * 8, krow = tid / KCH;
  const int dp = tid % DP, kg = tid / DP;

#define DSV4_FILL(mc_, buf_)                                                                   \
  do {                                                                                         \
    if (tid < MC) {                                                                            \
      const uint16_t *kp_, *vp_;                                                               \
      const bool ok_ = key_ptrs(a, bq, kr, s0 + (int64_t)(mc_) * MC + tid, &kp_, &vp_);         \
      kptr[buf_][tid] = kp_;                                                                   \
      vptr[buf_][tid] = vp_;                                                                   \
      const uint64_t m_ = __ballot(ok_);                                                       \
      if (lane == 0) {                                                                         \
        valid[buf_][2 * wave] = (uint32_t)m_;                                                  \
        valid[buf_][2 * wave + 1] = (uint32_t)(m_ >> 32);                                      \
      }                                                                                        \
    }                                                                                          \
  } while (0)
#define DSV4_LOAD_K(buf_, t_)                                                                  \
  do {                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < KLD; ++i_) {                                       \
      const uint4 v_ = gload_u4(kptr[buf_][(t_) * kTile + krow + i_ * KROWS] + kcol);          \
      reg[4 * i_] = v_.x; reg[4 * i_ + 1] = v_.y; reg[4 * i_ + 2] = v_.z; reg[4 * i_ + 3] = v_.w; \
    }                                                                                          \
  } while (0)
#define DSV4_LOAD_V(buf_, t_)                                                                  \
  do {                                                                                         \
    _Pragma("unroll") for (int e_ = 0; e_ < KPG; ++e_)                                         \
      reg[e_] = gload_u32(vptr[buf_][(t_) * kTile + kg * KPG + e_] + 2 * dp);                  \
  } while (0)

  if (nmacro > 0) {
    DSV4_FILL(0, 0);
    __syncthreads();
    DSV4_LOAD_K(0, 0);
  }
  for (int mc = 0; mc < nmacro; ++mc) {
    const int buf = mc & 1;
    const int64_t left = s1 - s0 - (int64_t)mc * MC;
    const int ntile = left < MC ? (int)((left + kTile - 1) / kTile) : TPM;
    // ---- phase K: scores of every key of the macro-chunk (S^T = K . Q^T)
    f32x4 s[TPM][2];
#pragma unroll
    for (int t = 0; t < TPM; ++t) {
      s[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < ntile) {
        __syncthreads();                   // the previous tile's LDS reads are done
#pragma unroll
        for (int i = 0; i < KLD; ++i)
          *reinterpret_cast<uint4*>(&tile[(krow + i * KROWS) * KSTR + kcol]) =
              make_uint4(reg[4 * i], reg[4 * i + 1], reg[4 * i + 2], reg[4 * i + 3]);
        __syncthreads();
        if (t + 1 < ntile) DSV4_LOAD_K(buf, t + 1);
        else DSV4_LOAD_V(buf, 0);
        if (wave_on) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const uint16_t* kr_l = &tile[(kt * 16 + col) * KSTR + g * (D / 4)];
#pragma unroll
            for (int c = 0; c < KS; ++c) {
              const uint4 kv = *reinterpret_cast<const uint4*>(kr_l + 8 * c);
              s[t][kt] = mfma_bf16(bit_cast_to<bf16x8>(kv), bit_cast_to<bf16x8>(qop[c]), s[t][kt]);
            }
          }
        }
      }
    }
    if (mc + 1 < nmacro) DSV4_FILL(mc + 1, buf ^ 1);
    // ---- softmax over the macro-chunk for head `head` (lane: keys 16kt+4g+i of each tile)
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPM; ++t) {
      const uint32_t vm = t < ntile ? valid[buf][t] : 0u;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (vm >> (kt * 16 + 4 * g + i)) & 1u;
          s[t][kt][i] = ok ? s[t][kt][i] * sl2 : -INFINITY;
          mx = fmaxf(mx, s[t][kt][i]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (m_run != -INFINITY && m_new > m_run) {
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
    }
    m_run = m_new;
    uint4 pop[TPM];
#pragma unroll
    for (int t = 0; t < TPM; ++t) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(s[t][0][i] - m_use);
        p[4 + i] = exp2f(s[t][1][i] - m_use);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) l_run += p[i];
      pop[t] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7]));
    }
    // ---- phase V: O^T += V^T . P^T
#pragma unroll
    for (int t = 0; t < TPM; ++t) {
      if (t < ntile) {
        __syncthreads();
#pragma unroll
        for (int e8 = 0; e8 < KPG; e8 += 8) {
          uint4 lo, hi;
          lo.x = __builtin_amdgcn_perm(reg[e8 + 1], reg[e8 + 0], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(reg[e8 + 3], reg[e8 + 2], 0x05040100u);
          lo.z = __builtin_amdgcn_perm(reg[e8 + 5], reg[e8 + 4], 0x05040100u);
          lo.w = __builtin_amdgcn_perm(reg[e8 + 7], reg[e8 + 6], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(reg[e8 + 1], reg[e8 + 0], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(reg[e8 + 3], reg[e8 + 2], 0x07060302u);
          hi.z = __builtin_amdgcn_perm(reg[e8 + 5], reg[e8 + 4], 0x07060302u);
          hi.w = __builtin_amdgcn_perm(reg[e8 + 7], reg[e8 + 6], 0x07060302u);
          const int key0 = kg * KPG + e8;
          *reinterpret_cast<uint4*>(&tile[(2 * dp) * VSTR + key0]) = lo;
          *reinterpret_cast<uint4*>(&tile[(2 * dp + 1) * VSTR + key0]) = hi;
        }
        __syncthreads();
        if (t + 1 < ntile) DSV4_LOAD_V(buf, t + 1);
        else if (mc + 1 < nmacro) DSV4_LOAD_K(buf ^ 1, 0);
        if (wave_on) {
          const bf16x8 pb = bit_cast_to<bf16x8>(pop[t]);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const uint16_t* vr = &tile[(dt * 16 + col) * VSTR + 4 * g];
            const uint2 lo = *reinterpret_cast<const uint2*>(vr);
            const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
            acc[dt] = mfma_bf16(bit_cast_to<bf16x8>(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[dt]);
          }
        }
      }
    }
  }
#undef DSV4_FILL
#undef DSV4_LOAD_K
#undef DSV4_LOAD_V

  if (!wave_on) return;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  const int64_t R = a.B * a.Q * a.H;
  const int64_t orow = bq * a.H + head;
  if (splits == 1) {
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + orow * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(out + dt * 16 + 4 * g) = w;
    }
    if (g == 0 && a.lse) a.lse[orow] = lse;
  } else {
    float* op = o_part + ((int64_t)split * R + orow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(op + dt * 16 + 4 * g) =
          make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
    if (g == 0) lse_part[(int64_t)split * R + orow] = lse;
  }
}

// ---------------------------------------------------------------------------- fp32 / VALU
__global__ __launch_bounds__(kThreads) void attend_f32_kernel(AttendArgs a) {
  extern __shared__ float fsm[];
  float* qs = fsm;                       // [D]
  float* ps = fsm + a.D;                 // [kThreads]
  __shared__ const float* kp[kThreads];
  __shared__ const float* vp[kThreads];
  __shared__ float red[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bq = blockIdx.y;
  const int h = blockIdx.x;
  const int D = a.D;
  const KeyRange kr = key_range(a, bq);
  const float* kc = reinterpret_cast<const float*>(a.kc);
  const float* vc = reinterpret_cast<const float*>(a.vc);
  const float* kw = reinterpret_cast<const float*>(a.kw);
  const float* vw = reinterpret_cast<const float*>(a.vw);
  for (int d = tid; d < D; d += kThreads) qs[d] = reinterpret_cast<const float*>(a.q)[(bq * a.H + h) * D + d];
  float acc[2] = {0.f, 0.f};             // dims tid, tid + 256
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t base = 0; base < kr.n_tot; base += kThreads) {
    __syncthreads();
    int64_t pos = base + tid;
    bool win = false;
    int64_t off = pos < kr.n_tot ? key_row(a, bq, kr, pos, &win) : -1;
    kp[tid] = off >= 0 ? (win ? kw : kc) + off : nullptr;
    vp[tid] = off >= 0 ? (win ? vw : vc) + off : nullptr;
    float s = -INFINITY;
    if (off >= 0) {
      const float* k = kp[tid];
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 = fmaf(qs[d], k[d], d0);
      s = d0 * a.scale;
    }
    float mx = wave_max(s);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, mx);
    float p = (m_new == -INFINITY || s == -INFINITY) ? 0.f : expf(s - m_new);
    ps[tid] = p;
    float sum = wave_sum(p);
    if (lane == 0) red[4 + wave] = sum;
    __syncthreads();
    sum = red[4] + red[5] + red[6] + red[7];
    if (m_new != -INFINITY) {
      const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
      l_run = l_run * alpha + sum;
      m_run = m_new;
      int64_t cnt = kr.n_tot - base < kThreads ? kr.n_tot - base : kThreads;
      for (int j = 0; j < 2; ++j) {
        int d = tid + j * kThreads;
        if (d >= D) break;
        float v = acc[j] * alpha;
        for (int e = 0; e < cnt; ++e)
          if (vp[e]) v = fmaf(ps[e], vp[e][d], v);
        acc[j] = v;
      }
    }
  }
  const int64_t orow = bq * a.H + h;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int j = 0; j < 2; ++j) {
    int d = tid + j * kThreads;
    if (d < D) reinterpret_cast<float*>(a.out)[orow * D + d] = acc[j] * inv;
  }
  if (tid == 0 && a.lse) a.lse[orow] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

// ---------------------------------------------------------------------------- LSE merge
// One wave per output row: the part weights exp(lse_p - max) are formed with wave
// shuffles into a per-wave LDS slice, then every lane accumulates NV float4 columns over
// the parts, four parts at a time so that several loads are in flight.
template <int NV>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(const float* __restrict__ o_parts,
                                                             const float* __restrict__ lse_parts, int P, int64_t R,
                                                             int D, void* __restrict__ out, int out_f32,
                                                             float* __restrict__ lse_out) {
  __shared__ float wsh[kThreads / kWave][1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + wave;
  if (r >= R) return;                    // whole wave; no workgroup barrier below
  float* w = wsh[wave];
  float mx = -INFINITY;
  for (int p = lane; p < P; p += kWave) mx = fmaxf(mx, lse_parts[(int64_t)p * R + r]);
  mx = wave_max(mx);
  float tot = 0.f;
  for (int p = lane; p < P; p += kWave) {
    float e = (mx == -INFINITY) ? 0.f : expf(lse_parts[(int64_t)p * R + r] - mx);
    w[p] = e;
    tot += e;
  }
  tot = wave_sum(tot);                   // the shuffles also order the LDS writes above
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int nd4 = D / 4;
  float4 acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* base = reinterpret_cast<const float4*>(o_parts + r * D);
  const int64_t pstride = R * D / 4;     // float4 stride between parts
  int p = 0;
  for (; p + 4 <= P; p += 4) {
    float4 v[4][NV];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        int d4 = lane + i * kWave;
        v[u][i] = d4 < nd4 ? base[(int64_t)(p + u) * pstride + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float wu = w[p + u];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        acc[i].x = fmaf(wu, v[u][i].x, acc[i].x);
        acc[i].y = fmaf(wu, v[u][i].y, acc[i].y);
        acc[i].z = fmaf(wu, v[u][i].z, acc[i].z);
        acc[i].w = fmaf(wu, v[u][i].w, acc[i].w);
      }
    }
  }
  for (; p < P; ++p) {
    float wu = w[p];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int d4 = lane + i * kWave;
      if (d4 >= nd4) continue;
      float4 v = base[(int64_t)p * pstride + d4];
      acc[i].x = fmaf(wu, v.x, acc[i].x);
      acc[i].y = fmaf(wu, v.y, acc[i].y);
      acc[i].z = fmaf(wu, v.z, acc[i].z);
      acc[i].w = fmaf(wu, v.w, acc[i].w);
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int d4 = lane + i * kWave;
    if (d4 >= nd4) continue;
    float4 s = make_float4(acc[i].x * inv, acc[i].y * inv, acc[i].z * inv, acc[i].w * inv);
    if (out_f32) {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + r * D)[d4] = s;
    } else {
      uint2 o2;
      o2.x = pack_bf16x2(s.x, s.y);
      o2.y = pack_bf16x2(s.z, s.w);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + r * D)[d4] = o2;
    }
  }
  if (lane == 0 && lse_out) lse_out[r] = (tot > 0.f) ? mx + logf(tot) : -INFINITY;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

AttendPlan plan_attend(const AttendArgs& a) {
  AttendPlan p{1, 0, 0};
  const int64_t win = a.W < a.L ? a.W : a.L;
  const int64_t n_max = (a.csa ? (int64_t)a.k : a.N) + (win > 0 ? win : 0);
  if (a.f32 || n_max == 0) {
    p.chunk = (int)(n_max > 0 ? n_max : 1);
    return p;
  }
  const int64_t rows = a.B * a.Q;
  int64_t want = (kTargetWorkgroups + rows - 1) / rows;   // about one workgroup per CU
  int64_t max_splits = (n_max + kTile - 1) / kTile;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int64_t chunk = (n_max + want - 1) / want;
  chunk = ((chunk + kTile - 1) / kTile) * kTile;
  int64_t splits = (n_max + chunk - 1) / chunk;
  p.splits = (int)splits;
  p.chunk = (int)chunk;
  if (splits > 1) {
    const int64_t R = a.B * a.Q * a.H;
    p.ws_bytes = align256((size_t)splits * R * a.D * 4) + align256((size_t)splits * R * 4);
  }
  return p;
}

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p, void* ws, hipStream_t st) {
  const int64_t rows = a.B * a.Q;
  if (rows == 0) return hipSuccess;
  if (a.f32) {
    size_t smem = (size_t)(a.D + kThreads) * 4;
    DSV4_LAUNCH_MAIN(attend_f32_kernel, dim3((unsigned)a.H, (unsigned)rows), dim3(kThreads), smem, st, a);
    return hipGetLastError();
  }
  float* o_part = nullptr;
  float* lse_part = nullptr;
  const int64_t R = rows * a.H;
  if (p.splits > 1) {
    o_part = reinterpret_cast<float*>(ws);
    lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + align256((size_t)p.splits * R * a.D * 4));
  }
  dim3 grid((unsigned)p.splits, (unsigned)rows);
  switch (a.D) {
    case 128: DSV4_LAUNCH_MAIN(attend_bf16_kernel<128>, grid, dim3(kThreads), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part); break;
    case 256: DSV4_LAUNCH_MAIN(attend_bf16_kernel<256>, grid, dim3(kThreads), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part); break;
    default: DSV4_LAUNCH_MAIN(attend_bf16_kernel<512>, grid, dim3(kThreads), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_lse_merge(o_part, lse_part, p.splits, R, a.D, a.out, false, a.lse, st);
}

hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, int64_t R, int D, void* out,
                            bool out_f32, float* lse_out, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int rows_per_wg = kThreads / kWave;
  dim3 grid((unsigned)((R + rows_per_wg - 1) / rows_per_wg));
  const int nv = (D / 4 + kWave - 1) / kWave;
#define DSV4_MERGE(NVv) DSV4_LAUNCH_MAIN(lse_merge_kernel<NVv>, grid, dim3(kThreads), 0, st, o_parts, lse_parts, P, R, \
                                         D, out, out_f32 ? 1 : 0, lse_out)
  if (nv <= 1) DSV4_MERGE(1);
  else if (nv <= 2) DSV4_MERGE(2);
  else if (nv <= 4) DSV4_MERGE(4);
  else if (nv <= 8) DSV4_MERGE(8);
  else DSV4_MERGE(16);
#undef DSV4_MERGE
  return hipGetLastError();
}

}  // namespace dsv4
