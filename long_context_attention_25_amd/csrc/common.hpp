// Device-side helpers shared by the gfx950 kernels: storage-format conversions,
// order-preserving score keys, wave reductions and MFMA operand types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHistBits = 12;                 // top bits of a score key used by the first select pass
constexpr int kHistBins = 1 << kHistBits;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {   // nearest-even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to two bf16 (nearest-even, one v_cvt_pk_bf16_f32 on gfx950), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Loads through the global address space (the pointers come from kernel-argument structs
// or LDS, where the compiler cannot see that they are global).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload_u4(const void* p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t gload_u32(const void* p) {
  return *(const __attribute__((address_space(1))) uint32_t*)(p);
}

// Streaming loads for data a call reads exactly once (cache rows, indexer keys, when one
// workgroup per sequence reads them): the non-temporal hint keeps the stream from
// displacing reused data in L2 and the Infinity Cache, and on MI355X plain streaming
// reads run ~10-15 % faster with it (2 GiB read: ~6.9-7.0 TB/s against ~6.0-6.3 TB/s
// with ordinary loads).  Data that several workgroups of a call read (many queries per
// sequence) is loaded the ordinary way: there the caches serve the repeats.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t load_stream(const uint8_t* p) { return __builtin_nontemporal_load(p); }
// Butterfly steps across the 16-lane rows of a wave: the values of lanes l and l ^ 16
// (l ^ 32) are exchanged by the gfx950 permlane swaps, a VALU operation, instead of a
// shuffle routed through the LDS crossbar.  The swap returns the two values of a lane
// pair in a lane-dependent order; their max or sum is the same in both lanes.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool kNT> __device__ __forceinline__ uint4 load_key(const uint4* p) {
  if constexpr (kNT) return load_stream(p); else return *p;
}
template <bool kNT> __device__ __forceinline__ uint2 load_key(const uint2* p) {
  if constexpr (kNT) return load_stream(p); else return *p;
}
template <bool kNT> __device__ __forceinline__ uint32_t load_key(const uint32_t* p) {
  if constexpr (kNT) return load_stream(p); else return *p;
}
template <bool kNT> __device__ __forceinline__ uint32_t load_key(const uint8_t* p) {
  if constexpr (kNT) return load_stream(p); else return *p;
}

// ------------------------------------------------------------------ OCP fp8 e4m3
// Nearest-even on the 3-bit mantissa, saturating to +-448 (0x7e), NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (__uint_as_float(a) >= 448.0f) return sign | 0x7eu;
  uint32_t code;
  if (a >= 0x3c800000u) {                           // >= 2^-6: normal range
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);   // round away the low 20 mantissa bits
    code = ((((r >> 23) & 0xffu) - 120u) << 3) | ((r >> 20) & 7u);
  } else {                                          // subnormal: multiples of 2^-9
    code = (uint32_t)__float2int_rn(__uint_as_float(a) * 512.0f);
  }
  return sign | code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------ OCP E2M1 (MXFP4 element)
// Nearest-even on the grid {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating to 6; sign in bit 3.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  float a = fabsf(v);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Shared MXFP4 exponent of a 32-element group: floor(log2 amax) - 2, clamped to
// [-127, 127]; 0 for an all-zero group.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;   // floor(log2) for normals
  if (e < -126) e = -127;                                         // subnormal amax
  int x = e - 2;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// ------------------------------------------------------------------ score keys
// Monotone map float -> uint32 (larger score <=> larger key); -0 and +0 map together.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ barriers
// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global access (vmcnt(0)), which would drain the next tile's prefetch at
// each tile; this one waits for the wave's LDS operations and leaves global loads in
// flight.  Use it only where the data exchanged through the barrier lives in LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ wave helpers
// Wave-wide max / sum, the result in every lane: DPP moves inside each 16-lane row (lane ^ 1
// and lane ^ 2 by quad permutes, then the mirrored lane of the other quad and of the other
// half row), then the permlane swaps across rows; no step goes through the LDS crossbar.
// Every step combines a lane pair symmetrically, so all lanes end with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_move<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return add_xor32(add_xor16(v));
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_fp8(long a, long b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// Wait until every vector-memory operation of this wave (loads and stores) has completed.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8)); }

template <typename T>
__device__ __forceinline__ T bit_cast_to(const uint4& v) {
  return __builtin_bit_cast(T, v);
}

// ------------------------------------------------------------------ debug builds
// Built with -DDSV4_DEBUG, the kernels also check facts that the release build only
// enforces by clamping (counts and indices read back from the workspace, the local
// selection's staging) and caller inputs that it tolerates (index entries other than -1
// outside [0, N), negative query positions).  A failed check sets its bit in the flag word
// of its source file and the kernel goes on exactly as the release build does.
enum DebugBit : uint32_t {
  kDbgRangeCount = 1u << 0,   // a scan range's candidate count above its key count
  kDbgThreshold = 1u << 1,    // the threshold bin, or the count above it, out of range
  kDbgCandIndex = 1u << 2,    // a candidate's key index at or past the visible keys
  kDbgLocalMeta = 1u << 3,    // a chunk's kept or visible count above what it can hold
  kDbgLocalStage = 1u << 4,   // more keys at or above the kept bin than the chunk keeps
  kDbgIdxEntry = 1u << 5,     // an index entry outside [0, N) other than -1
  kDbgQueryPos = 1u << 6,     // a negative query position
};
#ifdef DSV4_DEBUG
namespace {
__device__ uint32_t g_debug_flags;
}
#define DSV4_DCHECK(cond, bit)                                            \
  do {                                                                    \
    if (!(cond)) atomicOr(&::dsv4::g_debug_flags, (uint32_t)(bit));       \
  } while (0)
// host: this source file's flags since the last read, cleared (all ones if unreadable)
#define DSV4_DEBUG_READER(fn)                                                            \
  uint32_t fn() {                                                                        \
    uint32_t v = 0, z = 0;                                                               \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof(v)) != hipSuccess ||   \
        hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &z, sizeof(z)) != hipSuccess)       \
      return 0xffffffffu;                                                                \
    return v;                                                                            \
  }
#else
#define DSV4_DCHECK(cond, bit) \
  do {                         \
  } while (0)
#define DSV4_DEBUG_READER(fn) \
  uint32_t fn() { return 0u; }
#endif

}  // namespace dsv4
