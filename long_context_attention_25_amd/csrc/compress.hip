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
#include "pool.hpp"

namespace dsv4 {

namespace {

using pool::compress_body;
using pool::kThreads;
using pool::PoolState;
using pool::XVec;

template <typename TX, int YDT>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const TX* __restrict__ x, const float* __restrict__ gate, const float* __restrict__ bias,
    int64_t T, int C, int m, int64_t nb_per_b, int64_t total_blocks, int64_t x_bs, int64_t y_bs,
    void* __restrict__ y, uint8_t* __restrict__ ysc, int lpr, int spb, int bpw, int cs) {
  __shared__ float part[kThreads * (XVec<TX>::N + 2)];
  compress_body<TX, YDT>(x, gate, bias, T, C, m, nb_per_b, total_blocks, x_bs, y_bs, y, ysc, lpr, spb, bpw, cs,
                         blockIdx.x, part);
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
  __shared__ float part[kThreads * (XVec<TX>::N + 2)];
  compress_body<TX, YDT>(win + (b * L + first) * C, win_gate + b * L + first, bias, m, C, m, 1, 1, 0, 0, yr, sr, lpr,
                         spb, bpw, cs, slice, part, x_new + b * C, gnew);
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
using pool::plan_split;

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
using PoolJob = pool::Job;

template <typename TX, int Y1, int Y2>
__global__ __launch_bounds__(kThreads) void compress2_kernel(PoolJob j1, PoolJob j2, const float* __restrict__ gate,
                                                             const float* __restrict__ bias, int64_t T, int m,
                                                             int64_t nb_per_b, int64_t total_blocks) {
  __shared__ float part[kThreads * (XVec<TX>::N + 2)];
  if ((int64_t)blockIdx.x < j1.grid)
    compress_body<TX, Y1>(reinterpret_cast<const TX*>(j1.x), gate, bias, T, j1.C, m, nb_per_b, total_blocks, j1.x_bs,
                          j1.y_bs, j1.y, j1.ysc, j1.lpr, j1.spb, j1.bpw, j1.cs, blockIdx.x, part);
  else
    compress_body<TX, Y2>(reinterpret_cast<const TX*>(j2.x), gate, bias, T, j2.C, m, nb_per_b, total_blocks, j2.x_bs,
                          j2.y_bs, j2.y, j2.ysc, j2.lpr, j2.spb, j2.bpw, j2.cs, (int64_t)blockIdx.x - j1.grid, part);
}

template <typename TX, int Y1, int Y2>
hipError_t launch2_t(const CompressArgs& a, const CompressArgs& b, hipStream_t st) {
  const PoolJob j1 = pool::make_job<TX, Y1>(a), j2 = pool::make_job<TX, Y2>(b);
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
