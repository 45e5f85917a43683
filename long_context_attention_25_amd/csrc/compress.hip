// Softmax-gated block pooling (KV compression) for gfx950.
//
// One compressed entry is the softmax(gate + positional bias)-weighted sum of a
// disjoint block of m raw tokens (honbul.tistory.com/221, "CSA: 압축한 뒤, 필요한
// 기억만 골라서 보기" and "HCA: 더 강하게 압축하고, 압축된 전체를 보기"; pogovet.com
// 상세 정리 §4: 4x for CSA and 128x for HCA, softmax-gated pooling with a learned
// positional bias).
//
// The pass is a pure HBM stream (about one flop per byte): every thread owns one
// 16-byte channel vector of a row, so a wave reads whole rows with dwordx4 loads;
// the rows of one block are spread over the workgroup's row slots and reduced in
// LDS; the output is rounded (bf16 / fp8 e4m3) or quantised (MXFP4, with the
// 32-channel amax taken across the lanes that share a group) in registers.
#include "common.hpp"
#include "launch.hpp"

namespace dsv4 {

namespace {

constexpr int kThreads = 256;

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
template <typename TX, int YDT>
__device__ __forceinline__ void compress_body(
    const TX* __restrict__ x, const float* __restrict__ gate, const float* __restrict__ bias,
    int64_t T, int C, int m, int64_t nb_per_b, int64_t total_blocks, int64_t x_bs, int64_t y_bs,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int lpr, int spb, int bpw, int cs, int64_t wg,
    const TX* __restrict__ last_row = nullptr, float last_gate = 0.f) {
  // last_row (one block only): row m-1 of the block and its gate are taken from here
  // instead of x / gate
  constexpr int V = XVec<TX>::N;
  __shared__ float part[kThreads * (V + 2)];          // states crossing waves (or all states)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t blk0 = (wg / cs) * bpw;                // cs workgroups share a block group,
  const int slice = (int)(wg % cs);                    // each on lpr of its channel vectors

  const int rs_total = kThreads / lpr;
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
    float* p = part + tid * (V + 2);
    p[0] = st.M;
    p[1] = st.s;
#pragma unroll
    for (int v = 0; v < V; ++v) p[2 + v] = st.a[v];
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

template <typename TX, int YDT>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const TX* __restrict__ x, const float* __restrict__ gate, const float* __restrict__ bias,
    int64_t T, int C, int m, int64_t nb_per_b, int64_t total_blocks, int64_t x_bs, int64_t y_bs,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int lpr, int spb, int bpw, int cs) {
  compress_body<TX, YDT>(x, gate, bias, T, C, m, nb_per_b, total_blocks, x_bs, y_bs, y, ysc, lpr, spb, bpw, cs,
                         blockIdx.x);
}

// One decode step of cache maintenance; workgroup (slice, b) owns lpr channel vectors of
// sequence b: it writes its part of the new token's row into ring row pos[b] mod L (and
// the gate, which every slice writes alike), and when the token completes a block of m
// it pools its channels of the block's rows (contiguous in the ring, L being a multiple
// of m) into compressed row (pos[b] + 1) / m - 1.  The pooling reads the block's earlier
// rows from the window (written by earlier calls) and the new row from x_new.
template <typename TX, int YDT>
__global__ __launch_bounds__(kThreads) void append_kernel(
    const TX* __restrict__ x_new, const float* __restrict__ gate_new, const int32_t* __restrict__ pos,
    TX* __restrict__ win, float* __restrict__ win_gate, int64_t L, int C, const float* __restrict__ bias, int m,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int64_t y_bs, int64_t N, int lpr, int spb, int bpw, int cs) {
  const int64_t b = blockIdx.y;
  const int slice = blockIdx.x;
  const int tid = threadIdx.x;
  // the position through the scalar path (constant address space, uniform address)
  const int64_t p = *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(pos + b));
  if (p < 0) return;
  const int64_t row = p % L;
  const float gnew = gate_new[b];
  {
    // one channel vector is 16 bytes for both input types
    const uint4* src = reinterpret_cast<const uint4*>(x_new + b * C) + (int64_t)slice * lpr;
    uint4* dst = reinterpret_cast<uint4*>(win + (b * L + row) * C) + (int64_t)slice * lpr;
    for (int i = tid; i < lpr; i += kThreads) dst[i] = src[i];
    if (tid == 0) win_gate[b * L + row] = gnew;
  }
  const int64_t blk = (p + 1) / m - 1;
  if ((p + 1) % m != 0 || blk >= N) return;
  const int64_t first = (p + 1 - m) % L;
  const int64_t yrow = b * y_bs + blk;
  uint8_t* yr = reinterpret_cast<uint8_t*>(y);
  uint8_t* sr = ysc;
  if constexpr (YDT == 0) yr += yrow * C * 4;
  else if constexpr (YDT == 1) yr += yrow * C * 2;
  else if constexpr (YDT == 2) yr += yrow * C;
  else if constexpr (YDT == 4) yr += yrow * (C + kFp8RopeDims);   // (the scale bytes are per call)
  else {
    yr += yrow * (C / 2);
    sr += yrow * (C / 32);
  }
  // the block's last row is the new token: read from x_new, so that the pooling does not
  // wait for the window write above
  compress_body<TX, YDT>(win + (b * L + first) * C, win_gate + b * L + first, bias, m, C, m, 1, 1, 0, 0, yr, sr, lpr,
                         spb, bpw, cs, slice, x_new + b * C, gnew);
}

template <typename TX, int YDT>
hipError_t launch_t(const CompressArgs& a, hipStream_t st) {
  constexpr int V = XVec<TX>::N;
  const int lpr_full = (int)(a.C / V);
  const int64_t nb = a.T / a.m;
  const int64_t total = a.B * nb;
  // Split the channels over cs workgroups while that adds parallelism (few blocks):
  // a slice keeps at least one MXFP4 group (32/V lanes) and whole lanes.
  const int min_lanes = (YDT == 3) ? 32 / V : 1;
  int cs = 1;
  while (true) {
    int lpr = lpr_full / cs;
    int rs = kThreads / lpr;
    int spb = a.m < rs ? a.m : rs;
    int64_t groups = (total + rs / spb - 1) / (rs / spb);
    if (groups * cs >= 256 || lpr % 2 || lpr / 2 < min_lanes || lpr / 2 > kThreads) break;
    cs *= 2;
  }
  const int lpr = lpr_full / cs;
  const int rs = kThreads / lpr;
  const int spb = a.m < rs ? a.m : rs;
  const int bpw = rs / spb;
  const int64_t grid = ((total + bpw - 1) / bpw) * cs;
  DSV4_LAUNCH_MAIN((compress_kernel<TX, YDT>), dim3((unsigned)grid), dim3(kThreads), 0, st,
                   reinterpret_cast<const TX*>(a.x), a.gate, a.bias, a.T, (int)a.C, a.m, nb, total,
                   a.x_bs, a.y_bs, a.y, a.y_scale, lpr, spb, bpw, cs);
  return hipGetLastError();
}

// Channel split of the pooling: as for csa_compress (one block per sequence here).
template <typename TX, int YDT>
void plan_split(int64_t C, int m, int64_t blocks, int* lpr_o, int* spb_o, int* bpw_o, int* cs_o) {
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
hipError_t launch_append_t(const AppendArgs& a, hipStream_t st) {
  int lpr, spb, bpw, cs;
  plan_split<TX, YDT>(a.C, a.m, a.B, &lpr, &spb, &bpw, &cs);
  hipLaunchKernelGGL((append_kernel<TX, YDT>), dim3((unsigned)cs, (unsigned)a.B), dim3(kThreads), 0, st,
                     reinterpret_cast<const TX*>(a.x_new), a.gate_new, a.pos, reinterpret_cast<TX*>(a.win), a.win_gate,
                     a.L, (int)a.C, a.bias, a.m, a.y, a.y_scale, a.y_bs, a.N, lpr, spb, bpw, cs);
  return hipGetLastError();
}

// Two pooling jobs over the same raw blocks (same gates, bias, m and batch) in one launch,
// e.g. a CSA layer's K|V rows and its indexer key: workgroups [0, grid of job 1) run the
// first job with its own channel split, the rest the second.
struct PoolJob {
  const void* x;
  void* y;
  uint8_t* ysc;
  int64_t x_bs, y_bs;
  int C, lpr, spb, bpw, cs;
  int64_t grid;
};

template <typename TX, int Y1, int Y2>
__global__ __launch_bounds__(kThreads) void compress2_kernel(PoolJob j1, PoolJob j2, const float* __restrict__ gate,
                                                             const float* __restrict__ bias, int64_t T, int m,
                                                             int64_t nb_per_b, int64_t total_blocks) {
  if ((int64_t)blockIdx.x < j1.grid)
    compress_body<TX, Y1>(reinterpret_cast<const TX*>(j1.x), gate, bias, T, j1.C, m, nb_per_b, total_blocks, j1.x_bs,
                          j1.y_bs, j1.y, j1.ysc, j1.lpr, j1.spb, j1.bpw, j1.cs, blockIdx.x);
  else
    compress_body<TX, Y2>(reinterpret_cast<const TX*>(j2.x), gate, bias, T, j2.C, m, nb_per_b, total_blocks, j2.x_bs,
                          j2.y_bs, j2.y, j2.ysc, j2.lpr, j2.spb, j2.bpw, j2.cs, (int64_t)blockIdx.x - j1.grid);
}

template <typename TX, int YDT>
PoolJob pool_job(const CompressArgs& a) {
  PoolJob j;
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

template <typename TX, int Y1, int Y2>
hipError_t launch2_t(const CompressArgs& a, const CompressArgs& b, hipStream_t st) {
  const PoolJob j1 = pool_job<TX, Y1>(a), j2 = pool_job<TX, Y2>(b);
  DSV4_LAUNCH_MAIN((compress2_kernel<TX, Y1, Y2>), dim3((unsigned)(j1.grid + j2.grid)), dim3(kThreads), 0, st, j1,
                   j2, a.gate, a.bias, a.T, a.m, a.T / a.m, a.total_blocks());
  return hipGetLastError();
}

}  // namespace

// (bf16 x) K|V rows as bf16 or FP8 K|V rows, indexer key as MXFP4; checked by the caller
hipError_t launch_compress2(const CompressArgs& a, const CompressArgs& b, hipStream_t st) {
  if (a.total_blocks() == 0) return hipSuccess;
  if (a.y_dt == 4) return launch2_t<uint16_t, 4, 3>(a, b, st);
  return launch2_t<uint16_t, 1, 3>(a, b, st);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (a.total_blocks() == 0) return hipSuccess;
  if (a.x_f32) {
    switch (a.y_dt) {
      case 0: return launch_t<float, 0>(a, st);
      case 1: return launch_t<float, 1>(a, st);
      case 2: return launch_t<float, 2>(a, st);
      case 4: return launch_t<float, 4>(a, st);
      default: return launch_t<float, 3>(a, st);
    }
  }
  switch (a.y_dt) {
    case 0: return launch_t<uint16_t, 0>(a, st);
    case 1: return launch_t<uint16_t, 1>(a, st);
    case 2: return launch_t<uint16_t, 2>(a, st);
    case 4: return launch_t<uint16_t, 4>(a, st);
    default: return launch_t<uint16_t, 3>(a, st);
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.x_f32) {
    switch (a.y_dt) {
      case 0: return launch_append_t<float, 0>(a, st);
      case 1: return launch_append_t<float, 1>(a, st);
      case 2: return launch_append_t<float, 2>(a, st);
      case 4: return launch_append_t<float, 4>(a, st);
      default: return launch_append_t<float, 3>(a, st);
    }
  }
  switch (a.y_dt) {
    case 0: return launch_append_t<uint16_t, 0>(a, st);
    case 1: return launch_append_t<uint16_t, 1>(a, st);
    case 2: return launch_append_t<uint16_t, 2>(a, st);
    case 4: return launch_append_t<uint16_t, 4>(a, st);
    default: return launch_append_t<uint16_t, 3>(a, st);
  }
}

DSV4_DEBUG_READER(debug_flags_compress)

}  // namespace dsv4
