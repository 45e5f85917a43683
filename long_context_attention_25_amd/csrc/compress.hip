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

// YDT: 0 f32, 1 bf16, 2 fp8 e4m3, 3 MXFP4
template <typename TX, int YDT>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const TX* __restrict__ x, const float* __restrict__ gate, const float* __restrict__ bias,
    int64_t T, int C, int m, int64_t nb_per_b, int64_t total_blocks, int64_t x_bs, int64_t y_bs,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int lpr, int spb, int bpw, int cs) {
  constexpr int V = XVec<TX>::N;
  extern __shared__ float smem[];                      // weights [bpw*m] then partials [256*V]
  float* wts = smem;
  float* part = smem + bpw * m;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t blk0 = (int64_t)(blockIdx.x / cs) * bpw;   // cs workgroups share a block group,
  const int slice = blockIdx.x % cs;                         // each on lpr of its channel vectors

  // ---- this thread's first rows (up to 4) are loaded before the weights are computed,
  // so that the two memory round trips overlap
  const int rs_total = kThreads / lpr;
  const int slot = tid / lpr, cv = tid % lpr + slice * lpr;
  const int bi = slot / spb, r0 = slot % spb;
  const bool active = slot < rs_total && bi < bpw && blk0 + bi < total_blocks;
  const TX* xb = nullptr;
  float xf[4][V];
  if (active) {
    int64_t blk = blk0 + bi;
    int64_t b = blk / nb_per_b, i = blk % nb_per_b;
    xb = x + ((b * x_bs + i * m) * (int64_t)C) + (int64_t)cv * V;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (r0 + u * spb < m) XVec<TX>::load(xb + (int64_t)(r0 + u * spb) * C, xf[u]);
  }

  // ---- softmax weights of each block handled here, one wave per block
  for (int wi = wave; wi < bpw; wi += kThreads / kWave) {
    int64_t blk = blk0 + wi;
    if (blk >= total_blocks) break;
    int64_t b = blk / nb_per_b, i = blk % nb_per_b;
    const float* g = gate + b * T + i * m;
    float mx = -INFINITY;
    for (int j = lane; j < m; j += kWave) {
      float z = g[j] + bias[j];
      wts[wi * m + j] = z;
      mx = fmaxf(mx, z);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int j = lane; j < m; j += kWave) {
      float e = expf(wts[wi * m + j] - mx);
      wts[wi * m + j] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    float inv = 1.0f / sum;
    for (int j = lane; j < m; j += kWave) wts[wi * m + j] *= inv;
  }
  __syncthreads();

  // ---- weighted row sums: thread = (row slot, channel vector)
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  if (active) {
    const float* wb = wts + bi * m;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r0 + u * spb < m) {
        const float w = wb[r0 + u * spb];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = fmaf(w, xf[u][v], acc[v]);
      }
    }
    int j = r0 + 4 * spb;
    for (; j + 3 * spb < m; j += 4 * spb) {
      float xv[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) XVec<TX>::load(xb + (int64_t)(j + u * spb) * C, xv[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float w = wb[j + u * spb];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = fmaf(w, xv[u][v], acc[v]);
      }
    }
    for (; j < m; j += spb) {
      float xv[V];
      XVec<TX>::load(xb + (int64_t)j * C, xv);
      float w = wb[j];
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = fmaf(w, xv[v], acc[v]);
    }
  }
  if (spb > 1) {
    // combine the spb row slots of a block: a halving tree when spb is a power of two
#pragma unroll
    for (int v = 0; v < V; ++v) part[tid * V + v] = acc[v];
    __syncthreads();
    if ((spb & (spb - 1)) == 0) {
      for (int h = spb / 2; h >= 1; h >>= 1) {
        if (active && r0 < h) {
          const float* p = part + (tid + h * lpr) * V;
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] += p[v];
#pragma unroll
          for (int v = 0; v < V; ++v) part[tid * V + v] = acc[v];
        }
        __syncthreads();
      }
    } else if (active && r0 == 0) {
      for (int r = 1; r < spb; ++r) {
        const float* p = part + (tid + r * lpr) * V;
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += p[v];
      }
    }
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
  size_t smem = sizeof(float) * ((size_t)bpw * a.m + (size_t)kThreads * V);
  DSV4_LAUNCH_MAIN((compress_kernel<TX, YDT>), dim3((unsigned)grid), dim3(kThreads), smem, st,
                   reinterpret_cast<const TX*>(a.x), a.gate, a.bias, a.T, (int)a.C, a.m, nb, total,
                   a.x_bs, a.y_bs, a.y, a.y_scale, lpr, spb, bpw, cs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (a.total_blocks() == 0) return hipSuccess;
  if (a.x_f32) {
    switch (a.y_dt) {
      case 0: return launch_t<float, 0>(a, st);
      case 1: return launch_t<float, 1>(a, st);
      case 2: return launch_t<float, 2>(a, st);
      default: return launch_t<float, 3>(a, st);
    }
  }
  switch (a.y_dt) {
    case 0: return launch_t<uint16_t, 0>(a, st);
    case 1: return launch_t<uint16_t, 1>(a, st);
    case 2: return launch_t<uint16_t, 2>(a, st);
    default: return launch_t<uint16_t, 3>(a, st);
  }
}

}  // namespace dsv4
