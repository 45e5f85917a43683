// Measurement helpers for the benchmark, not part of the attention library: kernels that
// do nothing but stream HBM or issue MFMAs, so that the benchmark can state the rates
// this GPU reaches next to the published peaks (HBM 8 TB/s; dense MFMA 2.5 PFLOP/s bf16,
// 5 PFLOP/s fp8, 10.1 PFLOP/s fp4).  Built into libdsv4probe.so; only bench.py loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// Grid-stride read of n 16-byte words with the non-temporal hint (four loads in flight per
// lane); each thread stores the XOR of what it read so that the loads are kept.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                        uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// One MFMA of the given kind accumulating into c (a VGPR quad):
//   0: v_mfma_f32_16x16x32_bf16            1: v_mfma_f32_16x16x32_fp8_fp8
//   2: v_mfma_scale_f32_16x16x128_f8f6f4 with fp8 (e4m3) operands
//   3: the same with fp4 (e2m1) operands        4: v_mfma_f32_16x16x16_bf16
// Issued from asm so that the accumulators stay in place: compiled from the builtins, the
// loop below moved one of them through AGPR copies and padding every iteration, which
// halved the measured rate.
template <int KIND>
__device__ __forceinline__ void mfma_op(f32x4& c, const u32x4& a4, const i32x8& a8, uint32_t sc) {
  if constexpr (KIND == 0) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, %0" : "+v"(c) : "v"(a4));
  } else if constexpr (KIND == 1) {
    const uint64_t a2 = ((uint64_t)a4[1] << 32) | a4[0];
    asm volatile("v_mfma_f32_16x16x32_fp8_fp8 %0, %1, %1, %0" : "+v"(c) : "v"(a2));
  } else if constexpr (KIND == 2) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %1, %0, %2, %2 op_sel_hi:[0,0,0]"
                 : "+v"(c) : "v"(a8), "v"(sc));
  } else if constexpr (KIND == 3) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %1, %0, %2, %2 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                 : "+v"(c) : "v"(a4), "v"(sc));
  } else {
    const uint64_t a2 = ((uint64_t)a4[1] << 32) | a4[0];
    asm volatile("v_mfma_f32_16x16x16_bf16 %0, %1, %1, %0" : "+v"(c) : "v"(a2));
  }
}

// Eight independent accumulators per wave, used round-robin, so that an MFMA never waits
// on the one before it; operands come from the thread index so that nothing is folded.
template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int64_t iters, float* __restrict__ out) {
  const uint32_t w = 0x3c003c00u ^ (threadIdx.x & 0x00ff00ffu);   // small bf16 / fp8 / fp4 codes
  const u32x4 a4 = {w, w ^ 1u, w, w ^ 2u};
  const i32x8 a8 = {(int)w, (int)(w ^ 1u), (int)w, (int)w, (int)w, (int)w, (int)w, (int)w};
  const uint32_t sc = 127u;                                          // E8M0 scale 2^0
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int64_t it = 0; it < iters; ++it) {
    mfma_op<KIND>(c0, a4, a8, sc);
    mfma_op<KIND>(c1, a4, a8, sc);
    mfma_op<KIND>(c2, a4, a8, sc);
    mfma_op<KIND>(c3, a4, a8, sc);
    mfma_op<KIND>(c4, a4, a8, sc);
    mfma_op<KIND>(c5, a4, a8, sc);
    mfma_op<KIND>(c6, a4, a8, sc);
    mfma_op<KIND>(c7, a4, a8, sc);
  }
  // the MFMAs are opaque to the compiler: let them drain before the accumulators are read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `buf` once; `out` holds blocks * 256 words.
// Returns 0, or the HIP error code of the launch.
int dsv4probe_read(const void* buf, int64_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, out);
  return (int)hipGetLastError();
}

// Issues blocks * 4 waves * iters * 8 MFMAs of the given kind (0..4, see mfma_op); `out`
// holds blocks * 256 floats.  Flops per MFMA: 16*16*32*2 (kinds 0, 1), 16*16*128*2 (2, 3),
// 16*16*16*2 (4).
int dsv4probe_mfma(int kind, int64_t iters, float* out, int blocks, hipStream_t stream) {
  if (!out || iters <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out); break;
    case 1: hipLaunchKernelGGL(mfma_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out); break;
    case 2: hipLaunchKernelGGL(mfma_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out); break;
    case 3: hipLaunchKernelGGL(mfma_kernel<3>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out); break;
    case 4: hipLaunchKernelGGL(mfma_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, out); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
