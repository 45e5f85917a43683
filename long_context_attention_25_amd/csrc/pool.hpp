// Softmax-gated block pooling shared by the pooling kernels and by the indexer launch that
// also pools a decode step's newest block (compress_body below states the work split).
#ifndef DSV4_POOL_HPP
#define DSV4_POOL_HPP

#include "common.hpp"
#include "launch.hpp"

namespace dsv4 {
namespace pool {

constexpr int kThreads = 256;   // threads of a pooling workgroup

template <typename TX>
struct XVec;
template <>
struct XVec<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, float* o) {
    float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <>
struct XVec<uint16_t> {   // bf16
  static constexpr int N = 8;
  __device__ static void load(const void* p, float* o) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Running softmax-weighted sum over some rows of a block: with z_j = gate_j + bias_j,
// M = max z_j, s = sum exp(z_j - M) and a = sum exp(z_j - M) x_j; the pooled entry is
// a / s.  Two states of the same block combine exactly (up to rounding) by rescaling
// both to the larger maximum.
template <int V>
struct PoolState {
  float M, s, a[V];
  __device__ void init() {
    M = -INFINITY;
    s = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) a[v] = 0.f;
  }
  __device__ void add_rows(const float* z, const float (*x)[V], int n) {   // n <= 4 rows
    float mz = M;
    for (int u = 0; u < n; ++u) mz = fmaxf(mz, z[u]);
    const float f = M == -INFINITY ? 0.f : expf(M - mz);
    s *= f;
#pragma unroll
    for (int v = 0; v < V; ++v) a[v] *= f;
    for (int u = 0; u < n; ++u) {
      const float e = expf(z[u] - mz);
      s += e;
#pragma unroll
      for (int v = 0; v < V; ++v) a[v] = fmaf(e, x[u][v], a[v]);
    }
    M = mz;
  }
  __device__ void combine(float oM, float os, const float* oa) {
    const float mz = fmaxf(M, oM);
    if (mz == -INFINITY) return;                            // both empty
    const float f = expf(M - mz), g = expf(oM - mz);
    s = s * f + os * g;
#pragma unroll
    for (int v = 0; v < V; ++v) a[v] = a[v] * f + oa[v] * g;
    M = mz;
  }
};

// YDT: 0 f32, 1 bf16, 2 fp8 e4m3, 3 MXFP4, 4 FP8 K|V rows (the C channels are K then V of
// D = C/2 dims each; a row is K's first D - kFp8RopeDims channels as E4M3 codes, K's last
// kFp8RopeDims channels as bf16, then V as E4M3 codes: C + kFp8RopeDims bytes).  Codes
// are e4m3(y * 2^-e) with e = ysc[0] - 127 for K and ysc[1] - 127 for V (0 without ysc).
// Thread = (row slot, channel vector): slot r0 of a block takes rows r0, r0 + spb, ...
// and keeps a running state; the spb slots of a block are then combined.  When lpr and
// spb are powers of two the slots of a block sit at lane distances lpr, 2 lpr, ... and are
// combined by a butterfly within the wave, then (blocks wider than a wave) across waves
// through LDS; otherwise every state goes through LDS and the writer combines them.
// The work of workgroup `wg` (every thread of the workgroup calls it).
template <typename TX, int YDT, int NT = kThreads>
__device__ __forceinline__ void compress_body(
    const TX* __restrict__ x, const float* __restrict__ gate, const float* __restrict__ bias,
    int64_t T, int C, int m, int64_t nb_per_b, int64_t total_blocks, int64_t x_bs, int64_t y_bs,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int lpr, int spb, int bpw, int cs, int64_t wg,
    float* part, const TX* __restrict__ last_row = nullptr, float last_gate = 0.f, int tid = -1,
    float* y_lds = nullptr) {
  // NT: threads that pool.  part: LDS for the states that cross waves (NT * (V + 2) floats;
  // not touched when lpr * spb <= 64).  last_row (one block only): row m-1 of the block and
  // its gate are taken from here instead of x / gate.  tid: the thread's index in the
  // pooling (default threadIdx.x); threads at NT and above take part in the barriers only,
  // and a single wave may pool on its own (tid = lane) when lpr * spb <= 64 (no barrier
  // then).  y_lds (bf16 output, one block): the rounded values also go to LDS, at their
  // channel index, for a consumer in the same workgroup.
  constexpr int V = XVec<TX>::N;

  if (tid < 0) tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t blk0 = (wg / cs) * bpw;                // cs workgroups share a block group,
  const int slice = (int)(wg % cs);                    // each on lpr of its channel vectors

  const int rs_total = NT / lpr;
  const int slot = tid / lpr, cv = tid % lpr + slice * lpr;
  const int bi = slot / spb, r0 = slot % spb;
  const bool active = slot < rs_total && bi < bpw && blk0 + bi < total_blocks;
  PoolState<V> st;
  st.init();
  if (active) {
    const int64_t blk = blk0 + bi;
    const int64_t b = blk / nb_per_b, i = blk % nb_per_b;
    const TX* xb = x + ((b * x_bs + i * m) * (int64_t)C) + (int64_t)cv * V;
    const float* g = gate + b * T + i * m;
    // rows r0, r0 + spb, ... in groups of up to 4 (row and gate loads of a group together)
    for (int j = r0; j < m; j += 4 * spb) {
      float z[4];
      float xv[4][V];
      int n = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = j + u * spb;
        if (r < m) {
          if (last_row && r == m - 1) {
            XVec<TX>::load(last_row + (int64_t)cv * V, xv[u]);
            z[u] = last_gate + bias[r];
          } else {
            XVec<TX>::load(xb + (int64_t)r * C, xv[u]);
            z[u] = g[r] + bias[r];
          }
          n = u + 1;
        }
      }
      st.add_rows(z, xv, n);
    }
  }
  const bool pow2 = (lpr & (lpr - 1)) == 0 && (spb & (spb - 1)) == 0;
  if (pow2) {
    // butterfly over the slot bits inside the wave
    for (int d = lpr; d < kWave && d < lpr * spb; d <<= 1) {
      const float oM = __shfl_xor(st.M, d), os = __shfl_xor(st.s, d);
      float oa[V];
#pragma unroll
      for (int v = 0; v < V; ++v) oa[v] = __shfl_xor(st.a[v], d);
      st.combine(oM, os, oa);
    }
    if (lpr * spb > kWave) {
      // a block spans several waves: after the butterfly every group of g = 64/lpr slots
      // inside a wave (one slot when lpr >= 64) holds one state; the first slot of each
      // group stores it and the writer (slot 0) combines them
      const int g = lpr < kWave ? kWave / lpr : 1;
      if (active && r0 % g == 0) {
        float* p = part + tid * (V + 2);
        p[0] = st.M;
        p[1] = st.s;
#pragma unroll
        for (int v = 0; v < V; ++v) p[2 + v] = st.a[v];
      }
      __syncthreads();
      if (active && r0 == 0) {
        for (int r = g; r < spb; r += g) {
          const float* p = part + (tid + r * lpr) * (V + 2);
          st.combine(p[0], p[1], p + 2);
        }
      }
    }
  } else {
    if (tid < NT) {
      float* p = part + tid * (V + 2);
      p[0] = st.M;
      p[1] = st.s;
#pragma unroll
      for (int v = 0; v < V; ++v) p[2 + v] = st.a[v];
    }
    __syncthreads();
    if (active && r0 == 0) {
      for (int r = 1; r < spb; ++r) {
        const float* q = part + (tid + r * lpr) * (V + 2);
        st.combine(q[0], q[1], q + 2);
      }
    }
  }
  float acc[V];
  {
    const float inv = st.s > 0.f ? 1.f / st.s : 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = st.a[v] * inv;
  }
  const bool writer = active && r0 == 0;

  // ---- output rounding / quantisation
  int64_t blk = blk0 + bi;
  int64_t b = writer ? blk / nb_per_b : 0, i = writer ? blk % nb_per_b : 0;
  int64_t row = b * y_bs + i;
  if constexpr (YDT == 0) {
    if (writer) {
      float* yp = reinterpret_cast<float*>(y) + row * C + (int64_t)cv * V;
#pragma unroll
      for (int v = 0; v < V; ++v) yp[v] = acc[v];
    }
  } else if constexpr (YDT == 1) {
    if (writer) {
      uint32_t w[V / 2];
#pragma unroll
      for (int v = 0; v < V / 2; ++v) w[v] = pack_bf16x2(acc[2 * v], acc[2 * v + 1]);
      uint32_t* yp = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(y) + row * C + (int64_t)cv * V);
#pragma unroll
      for (int v = 0; v < V / 2; ++v) yp[v] = w[v];
      if (y_lds) {
#pragma unroll
        for (int v = 0; v < V / 2; ++v) {
          y_lds[cv * V + 2 * v] = __uint_as_float(w[v] << 16);
          y_lds[cv * V + 2 * v + 1] = __uint_as_float(w[v] & 0xffff0000u);
        }
      }
    }
  } else if constexpr (YDT == 2) {
    if (writer) {
      uint32_t w[V / 4];
#pragma unroll
      for (int v = 0; v < V / 4; ++v)
        w[v] = f32_to_e4m3(acc[4 * v]) | (f32_to_e4m3(acc[4 * v + 1]) << 8) |
               (f32_to_e4m3(acc[4 * v + 2]) << 16) | (f32_to_e4m3(acc[4 * v + 3]) << 24);
      uint32_t* yp = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(y) + row * C + (int64_t)cv * V);
#pragma unroll
      for (int v = 0; v < V / 4; ++v) yp[v] = w[v];
    }
  } else if constexpr (YDT == 4) {
    if (writer) {
      const int D = C / 2, DN = D - kFp8RopeDims;
      const int c0 = cv * V;                     // a vector never straddles a part
      uint8_t* yr = reinterpret_cast<uint8_t*>(y) + row * (int64_t)(C + kFp8RopeDims);
      if (c0 >= DN && c0 < D) {
        uint32_t w[V / 2];
#pragma unroll
        for (int v = 0; v < V / 2; ++v) w[v] = pack_bf16x2(acc[2 * v], acc[2 * v + 1]);
        uint32_t* yp = reinterpret_cast<uint32_t*>(yr + DN + 2 * (c0 - DN));
#pragma unroll
        for (int v = 0; v < V / 2; ++v) yp[v] = w[v];
      } else {
        const bool is_v = c0 >= D;
        const int e = ysc ? (int)ysc[is_v ? 1 : 0] - 127 : 0;
        uint32_t w[V / 4];
#pragma unroll
        for (int v = 0; v < V / 4; ++v)
          w[v] = f32_to_e4m3(ldexpf(acc[4 * v], -e)) | (f32_to_e4m3(ldexpf(acc[4 * v + 1], -e)) << 8) |
                 (f32_to_e4m3(ldexpf(acc[4 * v + 2], -e)) << 16) | (f32_to_e4m3(ldexpf(acc[4 * v + 3], -e)) << 24);
        uint32_t* yp = reinterpret_cast<uint32_t*>(yr + (is_v ? c0 + kFp8RopeDims : c0));
#pragma unroll
        for (int v = 0; v < V / 4; ++v) yp[v] = w[v];
      }
    }
  } else {
    // MXFP4: the 32 channels of a group live in 32/V consecutive lanes.
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) amax = fmaxf(amax, fabsf(acc[v]));
#pragma unroll
    for (int o = 1; o < 32 / V; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int X = mx_shared_exp(amax);
    uint32_t codes = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) codes |= f32_to_e2m1(ldexpf(acc[v], -X)) << (4 * v);
    if (writer) {
      uint8_t* yp = reinterpret_cast<uint8_t*>(y) + row * (C / 2) + (int64_t)cv * (V / 2);
      if constexpr (V == 8) *reinterpret_cast<uint32_t*>(yp) = codes;
      else *reinterpret_cast<uint16_t*>(yp) = (uint16_t)codes;
      if ((cv * V) % 32 == 0) ysc[row * (C / 32) + (cv * V) / 32] = (uint8_t)(X + 127);
    }
  }
}

// One pooling job over the blocks of a call: its channel split and its workgroup count.
struct Job {
  const void* x;
  void* y;
  uint8_t* ysc;
  int64_t x_bs, y_bs;
  int C, lpr, spb, bpw, cs;
  int64_t grid;
};

// Channel split of a job: cs workgroups share a group of blocks while that adds parallelism
// (few blocks); a slice keeps at least one MXFP4 group (32/V lanes) and whole lanes.
template <typename TX, int YDT>
inline void plan_split(int64_t C, int m, int64_t blocks, int* lpr_o, int* spb_o, int* bpw_o, int* cs_o) {
  constexpr int V = XVec<TX>::N;
  const int lpr_full = (int)(C / V);
  const int min_lanes = (YDT == 3) ? 32 / V : 1;
  int cs = 1;
  while (true) {
    int lpr = lpr_full / cs;
    int rs = kThreads / lpr;
    int spb = m < rs ? m : rs;
    int64_t groups = (blocks + rs / spb - 1) / (rs / spb);
    if (groups * cs >= 256 || lpr % 2 || lpr / 2 < min_lanes || lpr / 2 > kThreads) break;
    cs *= 2;
  }
  *lpr_o = lpr_full / cs;
  const int rs = kThreads / *lpr_o;
  *spb_o = m < rs ? m : rs;
  *bpw_o = rs / *spb_o;
  *cs_o = cs;
}

template <typename TX, int YDT>
inline Job make_job(const CompressArgs& a) {
  Job j;
  j.x = a.x;
  j.y = a.y;
  j.ysc = a.y_scale;
  j.x_bs = a.x_bs;
  j.y_bs = a.y_bs;
  j.C = (int)a.C;
  plan_split<TX, YDT>(a.C, a.m, a.total_blocks(), &j.lpr, &j.spb, &j.bpw, &j.cs);
  j.grid = ((a.total_blocks() + j.bpw - 1) / j.bpw) * j.cs;
  return j;
}

// The same job on as few workgroups as its results allow: when the planned split combines
// each block's slots inside one wave (power-of-two lpr and spb, lpr * spb <= 64), every
// such split with the same spb adds and combines the same values in the same order, so
// lpr = 64 / spb (one wave per block) gives the planned job's results bit for bit.  For
// a pooling that shares a launch with other work, where each workgroup waits for a slot.
template <typename TX, int YDT>
inline Job make_job_packed(const CompressArgs& a) {
  Job j = make_job<TX, YDT>(a);
  const int lpr_full = (int)(a.C / XVec<TX>::N);
  const int lpr = kWave / j.spb;
  const bool pow2 = (j.spb & (j.spb - 1)) == 0 && (j.lpr & (j.lpr - 1)) == 0;
  if (!pow2 || j.lpr * j.spb > kWave || lpr <= j.lpr || lpr > lpr_full || lpr_full % lpr != 0) return j;
  j.lpr = lpr;
  j.cs = lpr_full / lpr;
  j.bpw = (kThreads / lpr) / j.spb;
  j.grid = ((a.total_blocks() + j.bpw - 1) / j.bpw) * j.cs;
  return j;
}

}  // namespace pool
}  // namespace dsv4

#endif  // DSV4_POOL_HPP
