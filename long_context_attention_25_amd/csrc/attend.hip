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
// bf16 path (MQA: up to 64 query heads share one K/V row per key):
//   grid = (key-range splits, B*Q); one workgroup takes all heads of one query over one
//   key range, so each K/V byte crosses HBM once and is reused from LDS by every head.
//   The range is walked in 16-key tiles: K and V rows are copied straight into a
//   four-stage LDS ring (global_load_lds, three tiles in flight, rows padded so that
//   both operand read patterns are bank-conflict free).  S^T = K.Q^T comes from
//   mfma_f32_16x16x32_bf16 with K as the A operand, so each lane holds scores of one
//   head; exponentiated and rounded to bf16 they are directly the B operand of
//   O^T += V^T.P^T (mfma_f32_16x16x16_bf16, V^T read with transposing LDS reads).
//   Online softmax in fp32 (exp2 with the scale folded in; the hardware exp2, whose
//   arguments here are <= 0 or -inf) with lazy rescaling.  Splits write bf16 partial
//   outputs and fp32 lse that a merge kernel combines.
// bf16 query pairs (dense attention over many queries, e.g. a prefill chunk): two
//   queries per workgroup share every K/V tile copied into LDS; each wave serves one
//   query over the full head dim.
// FP8 K/V rows: the same scheme over E4M3 rows decoded in registers.
// fp32 path: a plain VALU kernel, one workgroup per (query, head).
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "pool.hpp"

namespace dsv4 {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;            // split granularity: key ranges are multiples of 32 keys
constexpr int kMaxCsaChunk = 2048;   // index entries of one CSA split (staged in LDS)
constexpr int64_t kMaxSplits = 1024;  // key-range splits per query (part weights held by the merge)
constexpr int kTargetWorkgroups = 256;   // gfx950: 256 CUs, one attention workgroup each
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;  // log2 units: rescale O only when the max grows by > 2^8
constexpr int kHeads = 64;            // query heads handled by one workgroup (4 head groups x 16)

struct KeyRange {
  int64_t n_c;      // compressed part length (CSA: k list slots, HCA: visible blocks)
  int64_t r_lo;     // first window row
  int64_t n_tot;    // n_c + window rows
};

// p: position of query bq, wp0: position of window row 0 of its sequence.  In ring mode
// (no win_pos0) wp0 is 0, window "rows" are absolute positions and wrow() maps them to
// buffer rows (position mod L); the caller keeps the last L >= W positions there.
__device__ __forceinline__ KeyRange key_range(const AttendArgs& a, int64_t p, int64_t wp0) {
  DSV4_DCHECK(p >= 0, kDbgQueryPos);
  KeyRange r;
  if (a.csa) {
    r.n_c = a.N > 0 ? a.k : 0;   // with no compressed entries every list slot is empty
  } else {
    int64_t n = p < 0 ? 0 : (p + 1) / a.m;
    r.n_c = n < a.N ? n : a.N;
  }
  int64_t lo = p - a.W + 1 - wp0;
  int64_t hi = p + 1 - wp0;
  if (lo < 0) lo = 0;
  if (a.win_pos0 && hi > a.L) hi = a.L;
  r.r_lo = lo;
  r.n_tot = r.n_c + (hi > lo ? hi - lo : 0);
  return r;
}
__device__ __forceinline__ KeyRange key_range(const AttendArgs& a, int64_t bq) {
  return key_range(a, a.q_pos[bq], a.win_pos0 ? a.win_pos0[bq / a.Q] : 0);
}
// Buffer row of window row r.
__device__ __forceinline__ int64_t wrow(const AttendArgs& a, int64_t r) { return a.win_pos0 ? r : r % a.L; }

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
    return (b * a.kv_bs + j) * a.kv_rs;
  }
  *win = true;
  return (b * a.L + wrow(a, kr.r_lo + (pos - kr.n_c))) * a.w_rs;
}

// ---------------------------------------------------------------------------- bf16 / MFMA
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

// Pointer held by lane `src` (src < 64): a scalar readlane when `src` is the same for the
// whole wave, a cross-lane shuffle otherwise.
template <bool kUniform, typename T>
__device__ __forceinline__ const T* lane_ptr(const T* p, int src) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  uint32_t lo, hi;
  if constexpr (kUniform) {
    lo = __builtin_amdgcn_readlane((uint32_t)v, src);
    hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
  } else {
    lo = (uint32_t)__shfl((int)(uint32_t)v, src);
    hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
  }
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Async copy of 16 bytes per lane from global memory (per-lane address) into LDS at byte
// address lds + 16 * lane; lds must be the same in every lane.  Issued from asm so that
// the compiler does not track it: it would otherwise make LDS reads wait for copies into
// other buffers.  The copy has no register result; completion is waited for explicitly
// with wait_vmcnt (it counts as a vector-memory operation until its data is in LDS).
// s_nop 3 covers the m0 write before the copy reads it.  kNT adds the non-temporal hint
// (nt), used for K/V rows that one workgroup of the call reads once (one query per
// sequence): such streams are faster with it and leave the caches to reused data.  It is
// a template parameter of the kernels: a branch per copy on a run-time flag cost ~2 us
// per decode launch.
template <bool kNT = false>
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
// A load through the constant address space: with a uniform address the compiler emits a
// scalar load, which the vector-memory counter does not track.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// Wait until at most n vector-memory operations of this wave are outstanding (n < 64).
// Copies into LDS count as vector-memory operations until their data is in LDS.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier for the tile ring: waits for this wave's LDS instructions only.  A
// fence-based barrier would also wait for every copy into LDS still in flight (they are
// LDS writes), i.e. for the next tile's prefetch; the copies a tile needs are waited for
// explicitly with wait_vmcnt before this barrier.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0xf) | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Launch shape of the HCA block pooling inside the attention launch (hca_pool_attend):
// grid rows at and past `rows` hold `grid` pooling workgroups, two per sequence (the K and
// the V half of the pooled entry), placed after the key-range workgroups so that they run
// on the CUs those leave free.
struct PoolLaunch {
  int64_t grid = 0;
  int rows = 0;
};

// One pooling workgroup: half `wg % 2` (K or V channels) of sequence b's pooled entry,
// rounded to bf16 into the cache row.  The K half then scores the entry for each of the
// sequence's queries and writes it as the last part of the split merge: lse = scale * q.k
// (-inf where the entry is not visible); the part's output, the entry's V row, is read by
// the merge from the cache row.  The pooling takes all NT threads: 64 lanes of 8 channels
// per row and NT / 64 row slots.
template <int D, int NT>
__device__ __forceinline__ void hca_pool_block(const AttendArgs& a, const PoolLaunch& pl, int part_ix,
                                               float* __restrict__ lse_part, float* lds) {
  const int64_t wg = (int64_t)(blockIdx.y - pl.rows) * gridDim.x + blockIdx.x;
  if (wg >= pl.grid) return;                                 // (whole workgroup)
  const int64_t b = wg / 2;
  const int half = (int)(wg % 2);
  constexpr int LPR = D / 8;                                 // lanes per row of one half
  constexpr int SPB = NT / LPR;
  static_assert(NT % LPR == 0 && (D / 8) * (SPB < 128 ? SPB : 128) <= NT, "pooling layout");
  uint16_t* yrow = reinterpret_cast<uint16_t*>(const_cast<void*>(a.kc)) + (b * a.kv_bs + a.pool.row) * a.kv_rs;
  float* krow = lds + NT * (pool::XVec<uint16_t>::N + 2);    // the rounded K half (D floats)
  pool::compress_body<uint16_t, 1, NT>(reinterpret_cast<const uint16_t*>(a.pool.x) + b * a.pool.x_bs * (2 * D),
                                       a.pool.gate + b * a.m, a.pool.bias, a.m, 2 * D, a.m, 1, 1, 0, 0, yrow, nullptr,
                                       LPR, a.m < SPB ? a.m : SPB, 1, 2, half, lds, nullptr, 0.f, -1,
                                       half == 0 ? krow : nullptr);
  if (half != 0) return;
  __syncthreads();
  const int64_t R = a.B * a.Q * a.H;
  constexpr int TPH = NT / 64;                               // threads per head (up to 64 heads)
  constexpr int DPT = D / TPH;                               // dims per thread
  const int h = threadIdx.x / TPH, j = threadIdx.x % TPH;
  for (int64_t qq = 0; qq < a.Q; ++qq) {
    const int64_t bq = b * a.Q + qq;
    const int64_t p = a.q_pos[bq];
    const int64_t nvis = p < 0 ? 0 : (p + 1) / a.m;
    float s = 0.f;
    if (h < a.H) {
      const uint4* qv = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + (bq * a.H + h) * D +
                                                       j * DPT);
      const float* kr = krow + j * DPT;
#pragma unroll
      for (int i = 0; i < DPT / 8; ++i) {
        const uint4 x = qv[i];
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = fmaf(__uint_as_float(xw[e] << 16), kr[8 * i + 2 * e], s);
          s = fmaf(__uint_as_float(xw[e] & 0xffff0000u), kr[8 * i + 2 * e + 1], s);
        }
      }
    }
#pragma unroll
    for (int o = 1; o < TPH; o <<= 1) s += __shfl_xor(s, o);
    if (h < a.H && j == 0) lse_part[(int64_t)part_ix * R + bq * a.H + h] = a.pool.row < nvis ? s * a.scale : -INFINITY;
  }
}

// One workgroup = 4 x DS waves: wave w owns heads 16(w%4) .. +15 and the slice w/4 of
// the head dim for the output (each of the DS waves of a head group computes the same
// scores over the full head dim; this keeps the accumulators in ordinary VGPRs).  The key list of the split is walked in 16-key tiles
// through a four-stage LDS ring: while tile t is used, tiles t+1 .. t+3 are being copied
// straight into LDS, so about 100 KB per CU stay in flight.  Rows are padded in LDS (K: +16
// bytes, V: +32 bytes) so that the K operand reads (16 rows, same column) and the
// transposed V reads (4 rows x 2 chunks per 16 lanes) hit distinct banks while every read
// of a lane uses one base address plus immediate offsets.
template <int D, int DS, bool kNT>
__global__ __launch_bounds__(kThreads * DS) void attend_bf16_kernel(AttendArgs a, int64_t chunk, int splits,
                                                               uint16_t* __restrict__ o_part,
                                                               float* __restrict__ lse_part, PoolLaunch pl) {
  constexpr int KT = 16;                   // keys per tile
  constexpr int NT = kThreads * DS;
  constexpr int NWV = NT / kWave;
  constexpr int KS = D / 32;               // MFMA k-steps over the head dim
  constexpr int DH = D / DS;               // output dims of a wave
  constexpr int NDT = DH / 16;             // 16-dim output tiles of a wave
  constexpr int RB = D * 2;                // bytes per row
  constexpr int KSTR = RB + 16;            // LDS row strides
  constexpr int VSTR = RB + 32;
  constexpr int LPR = RB / 16;             // lanes (16-byte chunks) per row
  constexpr int RPW = KT / NWV;            // rows copied per wave and matrix
  constexpr int NL = 2 * RPW;              // copy instructions per wave and tile
  constexpr int KTB = KT * KSTR, VTB = KT * VSTR;
  static_assert(LPR <= kWave && kWave % LPR == 0, "a row is copied by one instruction");
  static_assert(3 * NL < 64, "vmcnt range");

  constexpr int STB = KTB + VTB;          // one stage: K tile then V tile
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * STB];
  __shared__ int32_t list[kMaxCsaChunk];  // the split's index entries
  __shared__ __attribute__((aligned(16))) uint8_t xchg[DS > 1 ? 2 * NT * 16 : 16];   // partial scores, 2 buffers

  if (pl.grid > 0 && (int)blockIdx.y >= pl.rows) {          // the HCA block pooling workgroups
    if constexpr (D == 512) hca_pool_block<D, NT>(a, pl, splits, lse_part, reinterpret_cast<float*>(ring));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t bq = blockIdx.y;
  const int64_t b = bq / a.Q;
  const int split = blockIdx.x;
  const int64_t s0 = (int64_t)split * chunk;
  const int hg = wave % 4, dh = wave / 4;  // head group and output slice
  const int head = hg * 16 + col;
  const bool wave_on = hg * 16 < a.H;
  const bool direct = splits == 1 && pl.grid == 0;   // no merge: the output rows directly

  // The loads that do not depend on each other are issued together and waited for once:
  // the query position, the split's index entries (CSA: list slots s0 .. s0+chunk-1, all
  // below k <= n_tot), and the workgroup's query rows, copied once into LDS stages 2 and 3
  // (free until tile 2 is issued).  The copies into LDS are then the only vector-memory
  // operations in flight in the tile loop.
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t q_lds = ring_lds + 2 * STB;
  static_assert(kHeads * KSTR <= 2 * STB, "query rows fit in two stages");
  {
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + bq * a.H * D;
#pragma unroll
    for (int i = 0; i < kHeads / NWV; ++i) {
      const int h = wave + i * NWV;
      if (h < a.H && lane < LPR) copy16_to_lds(qb + h * D + lane * 8, q_lds + h * KSTR);
    }
  }
  const int64_t krs = a.kv_rs, wrs = a.w_rs;
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.kc) + b * a.kv_bs * krs;
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.vc) + b * a.kv_bs * krs;
  const uint16_t* kw = reinterpret_cast<const uint16_t*>(a.kw) + b * a.L * wrs;
  const uint16_t* vw = reinterpret_cast<const uint16_t*>(a.vw) + b * a.L * wrs;
  // Row pointers of a tile for key (lane % 16), set by tile_ptrs / spec_ptrs below.
  const uint16_t* my_kp;
  const uint16_t* my_vp;
  uint32_t vmask = 0;                       // validity of the tile's 16 keys
  // Wave w copies rows w, w+4, ... of the tile; a row is LPR lanes x 16 bytes (the other
  // lanes of a wave are masked off when a row is shorter than a wave).
  auto issue = [&](int stage) {
    const uint32_t kdst = ring_lds + stage * STB;
    const uint32_t vdst = kdst + KTB;
    const int j = lane / LPR;              // 0 unless LPR < 64
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = wave + i * NWV;
      const int off = (lane % LPR) * 8;
      if (j == 0) {
        copy16_to_lds<kNT>(lane_ptr<true>(my_kp, r) + off, kdst + r * KSTR);
        copy16_to_lds<kNT>(lane_ptr<true>(my_vp, r) + off, vdst + r * VSTR);
      }
    }
  };

  // HCA: tiles 0 and 1 are issued before the query position is known, as the compressed
  // rows s0 + ... (the rows they are, unless the split starts near the end of the visible
  // entries); they are checked below and issued again when wrong.
  const bool spec = !a.csa && a.N > 0;
  auto spec_ptrs = [&](int t) {
    int64_t j = s0 + (int64_t)t * KT + (lane & (KT - 1));
    if (j > a.N - 1) j = a.N - 1;
    my_kp = kc + j * krs;
    my_vp = vc + j * krs;
  };
  if (spec) {
    spec_ptrs(0);
    issue(0);
    spec_ptrs(1);
    issue(1);
  }
  const int32_t qpos = load_uniform(a.q_pos + bq);     // scalar loads: not counted by vmcnt
  const int32_t wpos0 = a.win_pos0 ? load_uniform(a.win_pos0 + b) : 0;
  constexpr int LPT = kMaxCsaChunk / NT;   // index entries per thread
  int32_t lv[LPT];
  const int64_t e1 = s0 + chunk < a.k ? s0 + chunk : a.k;
  // (each branch ends with its own wait, so that no load of one branch is seen as pending
  // in another)
  if (a.csa) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int64_t p = s0 + tid + u * NT;
      lv[u] = p < e1 ? a.idx[bq * a.k + p] : -1;
    }
    wait_vmcnt<0>();
  } else if (spec) {
    wait_vmcnt<2 * NL>();                   // the query rows (issued first) have landed
  } else {
    wait_vmcnt<0>();
  }
  const KeyRange kr = key_range(a, qpos, wpos0);
  int64_t s1 = s0 + chunk;
  if (s1 > kr.n_tot) s1 = kr.n_tot;
  const int ntile = s1 > s0 ? (int)((s1 - s0 + KT - 1) / KT) : 0;

  // CSA: the split's index entries, once, in LDS (the tile loop issues no other loads)
  if (a.csa) {
#pragma unroll
    for (int u = 0; u < LPT; ++u)
      if (s0 + tid + u * NT < e1) list[tid + u * NT] = lv[u];
  }
  __syncthreads();

  // Invalid slots point at a row that holds data (the query's first window row, else the
  // first compressed row), since their zero weights would not cancel a non-finite value.
  const bool win_rows = kr.n_tot > kr.n_c;
  const uint16_t* kdef = win_rows ? kw + wrow(a, kr.r_lo) * wrs : kc;
  const uint16_t* vdef = win_rows ? vw + wrow(a, kr.r_lo) * wrs : vc;
  auto tile_ptrs = [&](int t) {
    const int64_t pos = s0 + (int64_t)t * KT + (lane & (KT - 1));
    bool ok = false;
    const uint16_t* kp = kdef;
    const uint16_t* vp = vdef;
    if (pos < s1) {
      if (pos < kr.n_c) {
        const int64_t j = a.csa ? (int64_t)list[pos - s0] : pos;
        DSV4_DCHECK(j == -1 || (j >= 0 && j < a.N), kDbgIdxEntry);
        if (j >= 0 && j < a.N) {
          ok = true;
          kp = kc + j * krs;
          vp = vc + j * krs;
        }
      } else {
        const int64_t r = wrow(a, kr.r_lo + (pos - kr.n_c));
        ok = true;
        kp = kw + r * wrs;
        vp = vw + r * wrs;
      }
    }
    my_kp = kp;
    my_vp = vp;
    vmask = (uint32_t)__ballot(ok) & 0xffffu;
  };

  f32x4 acc[NDT];                          // O^T dims dh*DH + 16dt + 4g + i, head `head`
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  // Scores over the head dim are split between the DS waves of a head group: wave slice
  // dh takes k-steps dh*KSW .. +KSW-1 (dims g*D/4 + 8c .. +7 of lane group g for k-step c)
  // and the DS partial scores are summed through LDS.
  constexpr int KSW = KS / DS;
  // per-lane LDS byte offsets: K operand row `col` at this wave's first k-step; V^T rows
  // 4g + col/4 at dims dh*DH + 4(col%4)
  const int k_off = col * KSTR + g * (D / 4) * 2 + dh * KSW * 16;
  const int v_off = (4 * g + (col >> 2)) * VSTR + dh * DH * 2 + (col & 3) * 8;

  uint4 qop[KSW];                          // Q^T operands, read from LDS below
  // ---- partial S^T = K . Q^T (16 keys x 16 heads) over this wave's k-steps.  K operands
  // are read in batches of CB; batch i+1 is issued before the MFMAs of batch i (the
  // scheduling barriers keep the compiler from pairing each read with its MFMA; two
  // batches stay within the 15 outstanding LDS reads the counter tracks).  Two
  // accumulators halve the dependent MFMA chain.
  auto compute_s = [&](int stage) -> f32x4 {
    const uint8_t* kt_l = ring + stage * STB;
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
    constexpr int CB = KSW < 4 ? KSW : 4;
    constexpr int NB = KSW / CB;
    uint4 kv[2][CB];
    auto kread = [&](int buf, int c0) {
#pragma unroll
      for (int c = 0; c < CB; ++c) kv[buf][c] = *reinterpret_cast<const uint4*>(kt_l + k_off + (c0 + c) * 16);
    };
    kread(0, 0);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      if (bi + 1 < NB) kread((bi + 1) & 1, (bi + 1) * CB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        if ((bi * CB + c) & 1) sb = mfma_bf16(bit_cast_to<bf16x8>(kv[bi & 1][c]), bit_cast_to<bf16x8>(qop[bi * CB + c]), sb);
        else sa = mfma_bf16(bit_cast_to<bf16x8>(kv[bi & 1][c]), bit_cast_to<bf16x8>(qop[bi * CB + c]), sa);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return sa + sb;
  };
  // ---- softmax of the full scores (lane holds keys 4g + i of head `head`), lazy
  // rescaling, then O^T += V^T . P^T
  auto compute_pv = [&](int stage, uint32_t cur_mask, f32x4 s) {
    const uint8_t* vt_l = ring + stage * STB + KTB;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (cur_mask >> (4 * g + i)) & 1u;
      s[i] = ok ? s[i] * sl2 : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run + kLazyRescale) {
      if (m_run != -INFINITY) {
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i) acc[i] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
      l_run += pv[i];
    }
    // P^T operand of the 16x16x16 MFMA: this lane's own keys 4g .. 4g+3 of head `head`
    const v4i16 pb = __builtin_bit_cast(v4i16, make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])));
    // V^T operands by transposed LDS reads of the row-major tile: lane p of a 16-lane
    // block addresses key row 4g + p/4 at dims 16dt + 4(p%4) and receives its own dim
    // (16dt + p) from the four key rows.
    constexpr int DB = NDT < 4 ? NDT : 4;
    constexpr int ND = NDT / DB;
    v4i16 vt[2][DB];
    auto vread = [&](int buf, int d0) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
        vt[buf][d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(vt_l + v_off + (d0 + d) * 32));
    };
    vread(0, 0);
#pragma unroll
    for (int bi = 0; bi < ND; ++bi) {
      if (bi + 1 < ND) vread((bi + 1) & 1, (bi + 1) * DB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < DB; ++d)
        acc[bi * DB + d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[bi & 1][d], pb, acc[bi * DB + d], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile t lives in stage t % 4.  Tiles 0 and 1 are issued first; then every wave reads
  // its Q^T operands (head `head`, dims g*D/4 + 8c .. +7 for k-step c) from stages 2-3,
  // and after a barrier tile 2 is issued.  The scores of tile 0 are computed before the
  // loop; step t then waits for tile t+1 (tile t+2 stays in flight), passes one barrier
  // (tile t+1 visible to all waves; tile t's partial scores written; every wave done with
  // tile t-1), issues tile t+3 into the stage of tile t-1, sums tile t's partial scores,
  // computes the partial scores of tile t+1 and accumulates tile t's outputs: two
  // independent MFMA chains per step.  The partial scores alternate between two
  // exchange buffers (tile t in buffer t % 2).
  uint32_t mq0 = 0, mq1 = 0, mq2 = 0;      // masks of tiles t, t+1, t+2
  if (spec) {
    bool same = true;
    const uint16_t* sk[2];
    const uint16_t* sv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      spec_ptrs(t);
      sk[t] = my_kp;
      sv[t] = my_vp;
    }
    if (ntile > 0) {
      tile_ptrs(0);
      mq0 = vmask;
      same = same && __ballot(my_kp != sk[0] || my_vp != sv[0]) == 0;
    }
    if (ntile > 1) {
      tile_ptrs(1);
      mq1 = vmask;
      same = same && __ballot(my_kp != sk[1] || my_vp != sv[1]) == 0;
    }
    if (!same) {                             // copies of the right rows replace them
      wait_vmcnt<0>();
      if (ntile > 0) { tile_ptrs(0); issue(0); }
      if (ntile > 1) { tile_ptrs(1); issue(1); }
    }
  } else {
    if (ntile > 0) { tile_ptrs(0); mq0 = vmask; issue(0); }
    if (ntile > 1) { tile_ptrs(1); mq1 = vmask; issue(1); }
  }
  {
    const uint8_t* ql = ring + 2 * STB + (wave_on ? head : 0) * KSTR + g * (D / 4) * 2 + dh * KSW * 16;
#pragma unroll
    for (int c = 0; c < KSW; ++c) qop[c] = *reinterpret_cast<const uint4*>(ql + c * 16);
  }
  tile_barrier();
  if (ntile > 2) { tile_ptrs(2); mq2 = vmask; issue(2); }
  f32x4* xs = reinterpret_cast<f32x4*>(xchg);
  f32x4 sc_next = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ntile > 0) {
    if (ntile > 2) wait_vmcnt<2 * NL>();
    else if (ntile > 1) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    tile_barrier();
    if (wave_on) {
      sc_next = compute_s(0);
      if constexpr (DS > 1) xs[wave * kWave + lane] = sc_next;
    }
  }
  for (int t = 0; t < ntile; ++t) {
    if (t + 2 < ntile) wait_vmcnt<NL>();     // tile t+1 has landed (t+2 may be in flight)
    else wait_vmcnt<0>();
    tile_barrier();    // tile t+1 visible; tile t's partial scores written; tile t-1 done
    uint32_t mq3 = 0;
    if (t + 3 < ntile) {
      tile_ptrs(t + 3);
      mq3 = vmask;
      issue((t + 3) & 3);
    }
    f32x4 sc = sc_next;
    if constexpr (DS > 1) {
      if (wave_on) {
        const f32x4* xb = xs + (t & 1) * NT;
        f32x4 tot = xb[hg * kWave + lane];
#pragma unroll
        for (int j = 1; j < DS; ++j) tot += xb[(hg + 4 * j) * kWave + lane];
        sc = tot;
      }
    }
    if (wave_on && t + 1 < ntile) {
      sc_next = compute_s((t + 1) & 3);
      if constexpr (DS > 1) xs[((t + 1) & 1) * NT + wave * kWave + lane] = sc_next;
    }
    if (wave_on) compute_pv(t & 3, mq0, sc);
    mq0 = mq1;
    mq1 = mq2;
    mq2 = mq3;
  }
  wait_vmcnt<0>();                           // no copy into LDS outlives the workgroup
  __syncthreads();                           // every wave is done with the ring

  // the output rows, or with several splits this split's partial rows (bf16 like the
  // output; the merge accumulates in fp32): staged in LDS as [head][dim] rows, then
  // written with one 16-byte store per lane, a whole row per wave instruction (a lane's
  // accumulators hold 4 dims of one head: stored directly they make 32-byte pieces)
  constexpr int OSTR = RB + 16;              // staging row stride: the lanes' 8-byte writes hit distinct banks
  static_assert(kHeads * OSTR <= 4 * STB, "staged output rows fit in the ring");
  const int64_t R = a.B * a.Q * a.H;
  if (wave_on) {
    l_run = add_xor16(l_run);
    l_run = add_xor32(l_run);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    uint8_t* srow = ring + head * OSTR + (dh * DH + 4 * g) * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(srow + dt * 32) = w;
    }
    if (g == 0 && dh == 0) {
      const int64_t orow = bq * a.H + head;
      if (direct) {
        if (a.lse) a.lse[orow] = lse;
      } else {
        lse_part[(int64_t)split * R + orow] = lse;
      }
    }
  }
  __syncthreads();
  uint16_t* out = direct ? reinterpret_cast<uint16_t*>(a.out) + bq * a.H * D
                         : o_part + ((int64_t)split * R + bq * a.H) * D;
  const int nchunk = a.H * LPR;              // 16-byte chunks of the workgroup's rows
  for (int c = tid; c < nchunk; c += NT) {
    const int r = c / LPR, off = c % LPR;
    const uint4 v = *reinterpret_cast<const uint4*>(ring + r * OSTR + off * 16);
    *reinterpret_cast<uint4*>(out + (int64_t)r * D + off * 8) = v;
  }
}

// ---------------------------------------------------------------------------- FP8 K/V rows
// K rows of DN = D - kFp8RopeDims E4M3 codes followed by kFp8RopeDims bf16 values, V rows
// of D E4M3 codes.  Same work split as the bf16 kernel (D = 512: 8 waves, wave w owns
// heads 16(w%4) .. +15 and output dims (w/4)*256 .. +255), with 32-key tiles whose fp8
// rows are copied straight into a four-stage LDS ring (about 105 KB in flight per CU) and
// decoded exactly to bf16 in registers as MFMA operands are read:
//   S^T = K.Q^T per 16-key half: K operand = 8 code bytes of one key (one 8-byte LDS
//     read, four conversions) or 8 bf16 values for the RoPE dims; the k-steps take the
//     head dims in natural order (k-step c: dims 32c .. 32c+31) so that the bf16 dims
//     form whole k-steps, accumulated apart; k_scale multiplies the code dims' scores.
//   O^T += V^T.P^T with mfma_f32_16x16x32_bf16 over all 32 keys: a transposed 8-bit LDS
//     read gives a lane one dim of 8 keys (the 8 rows its 16-lane block addresses, two
//     lanes per row), chosen as the keys whose probabilities the lane already holds from
//     the two S^T halves (keys 4g..4g+3 and 16+4g..16+4g+3), so P^T needs no exchange.
//   v_scale multiplies the output.
// LDS rows are padded (K: +16 bytes, V: +16 bytes and +128 for the second half of a tile)
// so that the 8-byte K reads of 16 rows hit distinct banks and the two 16-lane blocks of
// a transposed V read that the LDS serves together (8 rows each) take disjoint halves of
// the banks.
constexpr int kListF8 = 512;          // index entries of one CSA split (FP8 kernel)

template <int D, bool kNT>
__global__ __launch_bounds__(kThreads * 2) void attend_fp8kv_kernel(AttendArgs a, int64_t chunk, int splits,
                                                                uint16_t* __restrict__ o_part,
                                                                float* __restrict__ lse_part) {
  constexpr int DS = 2;
  constexpr int KT = 32;                   // keys per tile
  constexpr int NT = kThreads * DS;
  constexpr int NWV = NT / kWave;
  constexpr int KS = D / 32;               // k-steps over the head dim
  constexpr int KSW = KS / DS;             // k-steps of a wave slice
  constexpr int DH = D / DS;               // output dims of a wave
  constexpr int NDT = DH / 16;             // 16-dim output tiles of a wave
  constexpr int DR = kFp8RopeDims, DN = D - DR;
  constexpr int KSR = DR / 32;             // bf16 k-steps: the last ones of slice DS-1
  constexpr int K8B = DN + 2 * DR, V8B = D;   // bytes of a K row and a V row
  constexpr int K8S = K8B + 16, V8S = V8B + 16;
  constexpr int VH = 128;                  // extra offset of V rows 16..31
  constexpr int KTB = KT * K8S, VTB = KT * V8S + VH;
  constexpr int STB = KTB + VTB;           // one stage: K tile then V tile
  constexpr int RPW = KT / NWV;            // rows copied per wave and matrix
  constexpr int NL = 2 * RPW;              // copy instructions per wave and tile
  constexpr int QSTR = 2 * D + 16;         // query rows in LDS
  static_assert(DS == 2 && KSR <= KSW && DN % 32 == 0, "slices and bf16 k-steps");
  static_assert(K8B % 16 == 0 && K8B / 16 <= kWave && V8B / 16 <= kWave, "one row per copy");
  static_assert(kHeads * QSTR <= 2 * STB, "query rows fit in two stages");
  static_assert(3 * NL < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * STB];
  __shared__ int32_t list[kListF8];
  __shared__ __attribute__((aligned(16))) f32x4 xchg[2 * NT];   // partial scores of both halves

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t bq = blockIdx.y;
  const int64_t b = bq / a.Q;
  const int split = blockIdx.x;
  const int64_t s0 = (int64_t)split * chunk;
  const int hg = wave % 4, dh = wave / 4;
  const int head = hg * 16 + col;
  const bool wave_on = hg * 16 < a.H;

  // query rows into stages 2 and 3 (free until tile 2 is issued), issued first
  const uint32_t ring_lds = lds_addr(ring);
  {
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + bq * a.H * D;
#pragma unroll
    for (int i = 0; i < kHeads / NWV; ++i) {
      const int h = wave + i * NWV;
      if (h < a.H && lane < D * 2 / 16) copy16_to_lds(qb + h * D + lane * 8, ring_lds + 2 * STB + h * QSTR);
    }
  }
  const int64_t krs = a.kv_rs, vrs = a.v_rs, wrs = a.w_rs, wvrs = a.wv_rs;   // bytes
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(a.kc) + b * a.kv_bs * krs;
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(a.vc) + b * a.kv_bs * vrs;
  const uint8_t* kw = reinterpret_cast<const uint8_t*>(a.kw) + b * a.L * wrs;
  const uint8_t* vw = reinterpret_cast<const uint8_t*>(a.vw) + b * a.L * wvrs;
  const uint8_t* my_kp;                    // row pointers of key (lane % 32) of a tile
  const uint8_t* my_vp;
  uint32_t vmask = 0;
  // Wave w copies rows w, w+8, w+16, w+24 of K and of V (one row per copy instruction).
  auto issue = [&](int stage) {
    const uint32_t kdst = ring_lds + stage * STB;
    const uint32_t vdst = kdst + KTB;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = wave + i * NWV;
      const uint8_t* kp = lane_ptr<true>(my_kp, r);
      const uint8_t* vp = lane_ptr<true>(my_vp, r);
      if (lane < K8B / 16) copy16_to_lds<kNT>(kp + lane * 16, kdst + r * K8S);
      if (lane < V8B / 16) copy16_to_lds<kNT>(vp + lane * 16, vdst + r * V8S + (r >= 16 ? VH : 0));
    }
  };
  // HCA: tiles 0 and 1 issued before the query position is known (checked below)
  const bool spec = !a.csa && a.N > 0;
  auto spec_ptrs = [&](int t) {
    int64_t j = s0 + (int64_t)t * KT + (lane & (KT - 1));
    if (j > a.N - 1) j = a.N - 1;
    my_kp = kc + j * krs;
    my_vp = vc + j * vrs;
  };
  if (spec) {
    spec_ptrs(0);
    issue(0);
    spec_ptrs(1);
    issue(1);
  }
  const int32_t qpos = load_uniform(a.q_pos + bq);
  const int32_t wpos0 = a.win_pos0 ? load_uniform(a.win_pos0 + b) : 0;
  static_assert(kListF8 % NT == 0, "list entries per thread");
  constexpr int LPT = kListF8 / NT;
  int32_t lv[LPT];
  const int64_t e1 = s0 + chunk < a.k ? s0 + chunk : a.k;
  if (a.csa) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int64_t p = s0 + tid + u * NT;
      lv[u] = p < e1 ? a.idx[bq * a.k + p] : -1;
    }
    wait_vmcnt<0>();
  } else if (spec) {
    wait_vmcnt<2 * NL>();                   // the query rows (issued first) have landed
  } else {
    wait_vmcnt<0>();
  }
  const KeyRange kr = key_range(a, qpos, wpos0);
  int64_t s1 = s0 + chunk;
  if (s1 > kr.n_tot) s1 = kr.n_tot;
  const int ntile = s1 > s0 ? (int)((s1 - s0 + KT - 1) / KT) : 0;
  if (a.csa) {
#pragma unroll
    for (int u = 0; u < LPT; ++u)
      if (s0 + tid + u * NT < e1) list[tid + u * NT] = lv[u];
  }
  __syncthreads();

  const bool win_rows = kr.n_tot > kr.n_c;
  const uint8_t* kdef = win_rows ? kw + wrow(a, kr.r_lo) * wrs : kc;
  const uint8_t* vdef = win_rows ? vw + wrow(a, kr.r_lo) * wvrs : vc;
  auto tile_ptrs = [&](int t) {
    const int64_t pos = s0 + (int64_t)t * KT + (lane & (KT - 1));
    bool ok = false;
    const uint8_t* kp = kdef;
    const uint8_t* vp = vdef;
    if (pos < s1) {
      if (pos < kr.n_c) {
        const int64_t j = a.csa ? (int64_t)list[pos - s0] : pos;
        DSV4_DCHECK(j == -1 || (j >= 0 && j < a.N), kDbgIdxEntry);
        if (j >= 0 && j < a.N) {
          ok = true;
          kp = kc + j * krs;
          vp = vc + j * vrs;
        }
      } else {
        const int64_t r = wrow(a, kr.r_lo + (pos - kr.n_c));
        ok = true;
        kp = kw + r * wrs;
        vp = vw + r * wvrs;
      }
    }
    my_kp = kp;
    my_vp = vp;
    vmask = (uint32_t)__ballot(ok);         // keys 0..31 (lanes 32..63 repeat them)
  };

  f32x4 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const float ksc = a.k_scale;
  uint4 qop[KSW];                          // Q^T operands: head `head`, dims 32(dh*KSW + c) + 8g .. +7

  auto cvt8 = [](uint32_t lo, uint32_t hi) -> bf16x8 {   // 8 E4M3 codes -> 8 bf16 (exact)
    const uint32_t w[4] = {
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true))};
    return bit_cast_to<bf16x8>(make_uint4(w[0], w[1], w[2], w[3]));
  };
  // ---- partial S^T (16 keys x 16 heads) of one 16-key half over this wave's k-steps.
  // kLast: slice DS-1, whose last KSR k-steps are the bf16 dims.
  auto compute_s = [&](const uint8_t* kt_l, int half, auto last_tag) -> f32x4 {
    constexpr bool kLast = decltype(last_tag)::value;
    constexpr int NC = kLast ? KSW - KSR : KSW;      // code k-steps of this slice
    const uint8_t* kb = kt_l + (half * 16 + col) * K8S + 8 * g + dh * KSW * 32;
    uint2 kx[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kx[c] = *reinterpret_cast<const uint2*>(kb + c * 32);
    uint4 kr4[KSR];
    if constexpr (kLast) {
      const uint8_t* rb = kt_l + (half * 16 + col) * K8S + DN + 16 * g;
#pragma unroll
      for (int c = 0; c < KSR; ++c) kr4[c] = *reinterpret_cast<const uint4*>(rb + c * 64);
    }
    f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa, sr = sa;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 ka = cvt8(kx[c].x, kx[c].y);
      if (c & 1) sb = mfma_bf16(ka, bit_cast_to<bf16x8>(qop[c]), sb);
      else sa = mfma_bf16(ka, bit_cast_to<bf16x8>(qop[c]), sa);
    }
    if constexpr (kLast) {
#pragma unroll
      for (int c = 0; c < KSR; ++c) sr = mfma_bf16(bit_cast_to<bf16x8>(kr4[c]), bit_cast_to<bf16x8>(qop[NC + c]), sr);
      return (sa + sb) * ksc + sr;
    }
    return (sa + sb) * ksc;
  };
  // V^T operand rows of this lane: its 16-lane block reads keys 4g .. 4g+3 and
  // 16+4g .. 16+4g+3 (lane pair (2i, 2i+1) one key row, 8 bytes each)
  const int vi = col >> 1;
  const int vrow = vi < 4 ? 4 * g + vi : 16 + 4 * g + (vi - 4);
  const int v_off = KTB + vrow * V8S + (vrow >= 16 ? VH : 0) + dh * DH + 8 * (col & 1);
  // ---- softmax over the 32 keys (lane: keys 4g+i and 16+4g+i of head `head`), lazy
  // rescaling, then O^T += V^T . P^T over the 32 keys
  auto compute_pv = [&](const uint8_t* st_l, uint32_t mask, f32x4 s0v, f32x4 s1v) {
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = ((mask >> (4 * g + i)) & 1u) ? s0v[i] * sl2 : -INFINITY;
      s[4 + i] = ((mask >> (16 + 4 * g + i)) & 1u) ? s1v[i] * sl2 : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, s[i]);
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run + kLazyRescale) {
      if (m_run != -INFINITY) {
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i) acc[i] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
      l_run += pv[i];
    }
    const bf16x8 pb = bit_cast_to<bf16x8>(make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                     pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])));
    constexpr int DB = 4;
    constexpr int ND = NDT / DB;
    v2i32 vt[2][DB];
    auto vread = [&](int buf, int d0) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
        vt[buf][d] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i32*)(st_l + v_off + (d0 + d) * 16));
    };
    vread(0, 0);
#pragma unroll
    for (int bi = 0; bi < ND; ++bi) {
      if (bi + 1 < ND) vread((bi + 1) & 1, (bi + 1) * DB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const v2i32 x = vt[bi & 1][d];
        acc[bi * DB + d] = mfma_bf16(cvt8((uint32_t)x.x, (uint32_t)x.y), pb, acc[bi * DB + d]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile t lives in stage t % 4; tiles 0 and 1 are issued first, the Q^T operands are read
  // from stages 2-3, then tile 2 is issued; step t waits for tile t, passes a barrier,
  // uses tile t and then issues tile t+3 into the stage of tile t-1.
  uint32_t mq0 = 0, mq1 = 0, mq2 = 0;
  if (spec) {
    bool same = true;
    const uint8_t* sk[2];
    const uint8_t* sv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      spec_ptrs(t);
      sk[t] = my_kp;
      sv[t] = my_vp;
    }
    if (ntile > 0) {
      tile_ptrs(0);
      mq0 = vmask;
      same = same && __ballot(my_kp != sk[0] || my_vp != sv[0]) == 0;
    }
    if (ntile > 1) {
      tile_ptrs(1);
      mq1 = vmask;
      same = same && __ballot(my_kp != sk[1] || my_vp != sv[1]) == 0;
    }
    if (!same) {
      wait_vmcnt<0>();
      if (ntile > 0) { tile_ptrs(0); issue(0); }
      if (ntile > 1) { tile_ptrs(1); issue(1); }
    }
  } else {
    if (ntile > 0) { tile_ptrs(0); mq0 = vmask; issue(0); }
    if (ntile > 1) { tile_ptrs(1); mq1 = vmask; issue(1); }
  }
  {
    const uint8_t* ql = ring + 2 * STB + (wave_on ? head : 0) * QSTR + 16 * g + dh * KSW * 64;
#pragma unroll
    for (int c = 0; c < KSW; ++c) qop[c] = *reinterpret_cast<const uint4*>(ql + c * 64);
  }
  tile_barrier();
  if (ntile > 2) { tile_ptrs(2); mq2 = vmask; issue(2); }
  for (int t = 0; t < ntile; ++t) {
    if (t + 2 < ntile) wait_vmcnt<2 * NL>();
    else if (t + 1 < ntile) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    tile_barrier();
    uint32_t mq3 = 0;
    const uint8_t* st_l = ring + (t & 3) * STB;
    f32x4 sc0 = f32x4{0.f, 0.f, 0.f, 0.f}, sc1 = sc0;
    if (wave_on) {
      if (dh == DS - 1) {
        sc0 = compute_s(st_l, 0, std::true_type{});
        sc1 = compute_s(st_l, 1, std::true_type{});
      } else {
        sc0 = compute_s(st_l, 0, std::false_type{});
        sc1 = compute_s(st_l, 1, std::false_type{});
      }
    }
    // partial scores of the two slices of a head group (waves hg and hg + 4), summed in
    // the same order by both
    if (wave_on) {
      xchg[wave * kWave + lane] = sc0;
      xchg[NT + wave * kWave + lane] = sc1;
    }
    tile_barrier();
    if (wave_on) {
      sc0 = xchg[hg * kWave + lane] + xchg[(hg + 4) * kWave + lane];
      sc1 = xchg[NT + hg * kWave + lane] + xchg[NT + (hg + 4) * kWave + lane];
      compute_pv(st_l, mq0, sc0, sc1);
    }
    if (t + 3 < ntile) {
      tile_ptrs(t + 3);
      mq3 = vmask;
      issue((t + 3) & 3);
    }
    mq0 = mq1;
    mq1 = mq2;
    mq2 = mq3;
  }
  wait_vmcnt<0>();
  __syncthreads();                           // every wave is done with the ring

  // output rows staged in LDS as [head][dim] bf16 rows, then one 16-byte store per lane
  constexpr int ORB = D * 2, OLPR = ORB / 16, OSTR = ORB + 16;
  static_assert(kHeads * OSTR <= 4 * STB, "staged output rows fit in the ring");
  const int64_t R = a.B * a.Q * a.H;
  if (wave_on) {
    l_run = add_xor16(l_run);
    l_run = add_xor32(l_run);
    const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
    const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    uint8_t* srow = ring + head * OSTR + (dh * DH + 4 * g) * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(srow + dt * 32) = w;
    }
    if (g == 0 && dh == 0) {
      const int64_t orow = bq * a.H + head;
      if (splits == 1) {
        if (a.lse) a.lse[orow] = lse;
      } else {
        lse_part[(int64_t)split * R + orow] = lse;
      }
    }
  }
  __syncthreads();
  uint16_t* out = splits == 1 ? reinterpret_cast<uint16_t*>(a.out) + bq * a.H * D
                              : o_part + ((int64_t)split * R + bq * a.H) * D;
  const int nchunk = a.H * OLPR;
  for (int c = tid; c < nchunk; c += NT) {
    const int r = c / OLPR, off = c % OLPR;
    const uint4 v = *reinterpret_cast<const uint4*>(ring + r * OSTR + off * 16);
    *reinterpret_cast<uint4*>(out + (int64_t)r * D + off * 8) = v;
  }
}

// ---------------------------------------------------------------------------- query pairs
// Dense (HCA) attention for many queries: a workgroup takes two queries of one sequence,
// whose key sets are the same but for at most one compressed entry and the window's
// ends when their positions are close (consecutive tokens of a prefill chunk), and walks
// the union of the two key lists once: every K/V tile is copied into LDS once for both.
// Wave w takes head group w%4 of query w/4 over the full head dim (Q^T operands 64 VGPRs,
// O^T accumulators 128), so no partial scores cross waves: no score exchange, each softmax
// computed once.  Per-query masks keep each query to its own keys.  The loop steps over
// 32 keys (two 16-key ring stages) per barrier so that P.V runs on the 16x16x32 MFMA.
// (Splitting the head dim between two waves instead, each wave serving both queries from
// one operand read, halves the LDS reads per flop but needs a score exchange and a second
// barrier per tile and computes every softmax twice: 2.2-2.3 ms against 1.74 ms for the
// 4096-query prefill layer.  One wave per SIMD serving 16 heads of both queries does not
// fit the register file: both queries' accumulators and Q^T operands spill.)
template <int D>
__global__ __launch_bounds__(kThreads * 2) void attend_bf16_pair_kernel(AttendArgs a, int64_t chunk, int splits,
                                                                        uint16_t* __restrict__ o_part,
                                                                        float* __restrict__ lse_part) {
  constexpr int KT = 16;
  constexpr int NT = kThreads * 2;
  constexpr int NWV = NT / kWave;          // 8
  constexpr int KS = D / 32;               // k-steps over the full head dim
  constexpr int NDT = D / 16;              // 16-dim output tiles over the full head dim
  constexpr int RB = D * 2;
  constexpr int KSTR = RB + 16;
  constexpr int VSTR = RB + 32;
  constexpr int LPR = RB / 16;
  constexpr int RPW = KT / NWV;
  constexpr int NL = 2 * RPW;
  constexpr int KTB = KT * KSTR, VTB = KT * VSTR;
  constexpr int STB = KTB + VTB;
  static_assert(LPR <= kWave && kWave % LPR == 0, "a row is copied by one instruction");
  static_assert(3 * NL < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * STB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t QP = (a.Q + 1) / 2;
  const int64_t b = blockIdx.y / QP;
  const int64_t q0 = (blockIdx.y % QP) * 2;
  const bool has1 = q0 + 1 < a.Q;
  const int64_t bq0 = b * a.Q + q0, bq1 = has1 ? bq0 + 1 : bq0;
  const int split = blockIdx.x;
  const int64_t s0 = (int64_t)split * chunk;
  const int hg = wave % 4, qi = wave / 4;  // head group, and which of the two queries
  const int head = hg * 16 + col;
  const bool wave_on = hg * 16 < a.H && (qi == 0 || has1);

  // Q^T operands of this wave's query straight into registers (dims g*D/4 + 8c .. +7 for
  // k-step c), waited for before any copy into LDS is issued
  uint4 qop[KS];
  {
    const int hh = wave_on ? head : 0;
    const int64_t bqw = qi == 0 ? bq0 : bq1;
    const uint4* pq = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + (bqw * a.H + hh) * D +
                                                     g * (D / 4));
#pragma unroll
    for (int c = 0; c < KS; ++c) qop[c] = pq[c];
  }
  const int32_t p0 = load_uniform(a.q_pos + bq0);
  const int32_t p1 = load_uniform(a.q_pos + bq1);
  const int32_t wpos0 = a.win_pos0 ? load_uniform(a.win_pos0 + b) : 0;
  wait_vmcnt<0>();
  // the union of the two key lists: compressed entries 0 .. n_c-1, then query 0's window
  // rows [lo0, hi0), then query 1's window rows outside that range, [lo1, min(hi1, lo0))
  // and [max(lo1, hi0), hi1) (window coordinates: buffer rows, or positions in ring
  // mode).  For neighbouring positions the second part is one row; it never exceeds W.
  const KeyRange k0 = key_range(a, p0, wpos0);
  const KeyRange k1 = has1 ? key_range(a, p1, wpos0) : k0;
  const int64_t lo0 = k0.r_lo, hi0 = k0.r_lo + (k0.n_tot - k0.n_c);
  const int64_t lo1 = k1.r_lo, hi1 = k1.r_lo + (k1.n_tot - k1.n_c);
  const int64_t e1a = hi1 < lo0 ? hi1 : lo0;               // end of [lo1, min(hi1, lo0))
  const int64_t nb1 = e1a > lo1 ? e1a - lo1 : 0;
  const int64_t s2 = lo1 > hi0 ? lo1 : hi0;                 // start of [max(lo1, hi0), hi1)
  const int64_t nb2 = hi1 > s2 ? hi1 - s2 : 0;
  const int64_t w0n = hi0 - lo0;
  const int64_t n_c = k0.n_c > k1.n_c ? k0.n_c : k1.n_c;
  const int64_t n_w = w0n + nb1 + nb2;
  const int64_t n_tot = n_c + n_w;
  auto wr_at = [&](int64_t pp) -> int64_t {                 // window coordinate of window entry pp
    return pp < w0n ? lo0 + pp : (pp < w0n + nb1 ? lo1 + (pp - w0n) : s2 + (pp - w0n - nb1));
  };
  int64_t s1 = s0 + chunk;
  if (s1 > n_tot) s1 = n_tot;
  const int ntile = s1 > s0 ? (int)((s1 - s0 + KT - 1) / KT) : 0;

  const int64_t krs = a.kv_rs, wrs = a.w_rs;
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.kc) + b * a.kv_bs * krs;
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.vc) + b * a.kv_bs * krs;
  const uint16_t* kw = reinterpret_cast<const uint16_t*>(a.kw) + b * a.L * wrs;
  const uint16_t* vw = reinterpret_cast<const uint16_t*>(a.vw) + b * a.L * wrs;
  // slots past the list point at a row that holds data
  const uint16_t* kdef = n_w > 0 ? kw + wrow(a, wr_at(0)) * wrs : kc;
  const uint16_t* vdef = n_w > 0 ? vw + wrow(a, wr_at(0)) * wrs : vc;
  const uint16_t* my_kp;
  const uint16_t* my_vp;
  uint32_t vm0 = 0, vm1 = 0;
  auto tile_ptrs = [&](int t) {
    const int64_t pos = s0 + (int64_t)t * KT + (lane & (KT - 1));
    bool ok0 = false, ok1 = false;
    const uint16_t* kp = kdef;
    const uint16_t* vp = vdef;
    if (pos < s1) {
      if (pos < n_c) {
        if (pos < a.N) {
          ok0 = pos < k0.n_c;
          ok1 = has1 && pos < k1.n_c;
          kp = kc + pos * krs;
          vp = vc + pos * krs;
        }
      } else {
        const int64_t r = wr_at(pos - n_c);
        ok0 = r >= lo0 && r < hi0;
        ok1 = has1 && r >= lo1 && r < hi1;
        const int64_t rr = wrow(a, r);
        kp = kw + rr * wrs;
        vp = vw + rr * wrs;
      }
    }
    my_kp = kp;
    my_vp = vp;
    vm0 = (uint32_t)__ballot(ok0) & 0xffffu;
    vm1 = (uint32_t)__ballot(ok1) & 0xffffu;
  };
  const uint32_t ring_lds = lds_addr(ring);
  auto issue = [&](int stage) {
    const uint32_t kdst = ring_lds + stage * STB;
    const uint32_t vdst = kdst + KTB;
    const int j = lane / LPR;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = wave + i * NWV;
      const int off = (lane % LPR) * 8;
      if (j == 0) {
        copy16_to_lds(lane_ptr<true>(my_kp, r) + off, kdst + r * KSTR);
        copy16_to_lds(lane_ptr<true>(my_vp, r) + off, vdst + r * VSTR);
      }
    }
  };

  f32x4 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int k_off = col * KSTR + g * (D / 4) * 2;
  const int v_off = (4 * g + (col >> 2)) * VSTR + (col & 3) * 8;

  // S^T of this wave's query over the full head dim for the two 16-key tiles of a step
  // (stages st and st + 1): 16 keys x 16 heads each, the two tiles' MFMAs interleaved so
  // that four accumulators carry the dependent chains
  auto compute_s2 = [&](int st, f32x4& s0, f32x4& s1) {
    const uint8_t* k0 = ring + st * STB + k_off;
    const uint8_t* k1 = k0 + STB;
    f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, b0 = a0, a1 = a0, b1 = a0;
    uint4 kv[2][2];
    auto kread = [&](int buf, int c) {
      kv[buf][0] = *reinterpret_cast<const uint4*>(k0 + c * 16);
      kv[buf][1] = *reinterpret_cast<const uint4*>(k1 + c * 16);
    };
    kread(0, 0);
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      if (c + 1 < KS) kread((c + 1) & 1, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 qb = bit_cast_to<bf16x8>(qop[c]);
      if (c & 1) {
        b0 = mfma_bf16(bit_cast_to<bf16x8>(kv[c & 1][0]), qb, b0);
        b1 = mfma_bf16(bit_cast_to<bf16x8>(kv[c & 1][1]), qb, b1);
      } else {
        a0 = mfma_bf16(bit_cast_to<bf16x8>(kv[c & 1][0]), qb, a0);
        a1 = mfma_bf16(bit_cast_to<bf16x8>(kv[c & 1][1]), qb, a1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 = a0 + b0;
    s1 = a1 + b1;
  };
  // softmax step of one query over a step's 32 keys: returns its P^T operand for the
  // 16x16x32 MFMA, k-slots 8g .. 8g+3 = keys 4g .. 4g+3 of the first tile and 8g+4 .. 8g+7
  // the same keys of the second (the rows a lane holds of each S^T tile)
  auto softmax2 = [&](uint32_t mk0, uint32_t mk1, f32x4 s0, f32x4 s1, float& m_run, float& l_run,
                      f32x4* acc) -> bf16x8 {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = ((mk0 >> (4 * g + i)) & 1u) ? s0[i] * sl2 : -INFINITY;
      s1[i] = ((mk1 >> (4 * g + i)) & 1u) ? s1[i] * sl2 : -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    }
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run + kLazyRescale) {
      if (m_run != -INFINITY) {
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i) acc[i] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p0[4], p1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = __builtin_amdgcn_exp2f(s0[i] - m_use);
      p1[i] = __builtin_amdgcn_exp2f(s1[i] - m_use);
      l_run += p0[i] + p1[i];
    }
    return bit_cast_to<bf16x8>(make_uint4(pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                                          pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])));
  };
  // O^T += V^T . P^T over the full head dim and a step's 32 keys on the 16x16x32 MFMA (the
  // 16x16x16 form runs at half its rate on gfx950): a lane's V^T operand is the transposed
  // read of its 4 keys from each of the two tiles, in the k-slot order of P^T
  auto compute_pv2 = [&](int st, bf16x8 pb) {
    const uint8_t* v0 = ring + st * STB + KTB + v_off;
    const uint8_t* v1 = v0 + STB;
    constexpr int DB = 2;
    constexpr int ND = NDT / DB;
    v4i16 vt[2][DB][2];
    auto vread = [&](int buf, int d0) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        vt[buf][d][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(v0 + (d0 + d) * 32));
        vt[buf][d][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(v1 + (d0 + d) * 32));
      }
    };
    vread(0, 0);
#pragma unroll
    for (int bi = 0; bi < ND; ++bi) {
      if (bi + 1 < ND) vread((bi + 1) & 1, (bi + 1) * DB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const uint2 lo = __builtin_bit_cast(uint2, vt[bi & 1][d][0]);
        const uint2 hi = __builtin_bit_cast(uint2, vt[bi & 1][d][1]);
        acc[bi * DB + d] = mfma_bf16(bit_cast_to<bf16x8>(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[bi * DB + d]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Steps of 32 keys: step u takes tiles 2u and 2u + 1, in stages 2(u % 2) and 2(u % 2) + 1.
  // Step u waits for its own two tiles and passes a barrier, after which every wave is done
  // with step u - 1, so step u + 1's tiles go into that step's stages before step u computes.
  const int nstep = (ntile + 1) / 2;
  uint32_t ca0 = 0, ca1 = 0, cb0 = 0, cb1 = 0;   // key masks of the current step's tiles (a: query 0, b: query 1)
  if (nstep > 0) {
    tile_ptrs(0); ca0 = vm0; cb0 = vm1; issue(0);
    tile_ptrs(1); ca1 = vm0; cb1 = vm1; issue(1);
  }
  for (int u = 0; u < nstep; ++u) {
    wait_vmcnt<0>();
    tile_barrier();
    uint32_t na0 = 0, na1 = 0, nb0 = 0, nb1 = 0;
    if (u + 1 < nstep) {
      const int st = ((u + 1) & 1) * 2;
      tile_ptrs(2 * u + 2); na0 = vm0; nb0 = vm1; issue(st);
      tile_ptrs(2 * u + 3); na1 = vm0; nb1 = vm1; issue(st + 1);
    }
    if (wave_on) {
      const int st = (u & 1) * 2;
      f32x4 sv0, sv1;
      compute_s2(st, sv0, sv1);
      const bf16x8 pb = softmax2(qi == 0 ? ca0 : cb0, qi == 0 ? ca1 : cb1, sv0, sv1, m_run, l_run, acc);
      compute_pv2(st, pb);
    }
    ca0 = na0; ca1 = na1;
    cb0 = nb0; cb1 = nb1;
  }
  wait_vmcnt<0>();
  __syncthreads();                           // every wave is done with the ring

  // both queries' output rows staged in LDS as [query][head][dim] bf16 rows, then one
  // 16-byte store per lane (the two rows of a head are consecutive in the output)
  constexpr int OSTR = RB + 16;
  static_assert(2 * kHeads * OSTR <= 4 * STB, "staged output rows fit in the ring");
  const int64_t R = a.B * a.Q * a.H;
  if (wave_on) {
    l_run = add_xor16(l_run);
    l_run = add_xor32(l_run);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    uint8_t* srow = ring + (qi * a.H + head) * OSTR + 4 * g * 2;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
      *reinterpret_cast<uint2*>(srow + dt * 32) = w;
    }
    if (g == 0 && (qi == 0 || has1)) {
      const int64_t orow = (bq0 + qi) * a.H + head;
      if (splits == 1) {
        if (a.lse) a.lse[orow] = lse;
      } else {
        lse_part[(int64_t)split * R + orow] = lse;
      }
    }
  }
  __syncthreads();
  uint16_t* out = splits == 1 ? reinterpret_cast<uint16_t*>(a.out) + bq0 * a.H * D
                              : o_part + ((int64_t)split * R + bq0 * a.H) * D;
  const int nchunk = (has1 ? 2 : 1) * a.H * LPR;   // rows of query 0, then of query 1
  for (int c = tid; c < nchunk; c += NT) {
    const int r = c / LPR, off = c % LPR;
    const uint4 v = *reinterpret_cast<const uint4*>(ring + r * OSTR + off * 16);
    *reinterpret_cast<uint4*>(out + (int64_t)r * D + off * 8) = v;
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

// Merge of the attention kernel's bf16 split partials (the arithmetic of lse_merge_kernel):
// one workgroup per output row.  Every wave computes the part weights exp(lse_p - lse)
// into its own LDS slice; wave w then accumulates parts w, w+4, ... for 8 dims per lane
// with up to 8 loads in flight, and the four partial sums are added through LDS.
constexpr int kMergePPT = 8;              // parts per lane and round
// extra_v (HCA pooling in the attention launch): part P-1 is a single entry whose output
// row is its V row, extra_v + (r / rows_per_seq) * extra_bs for output row r.
__global__ __launch_bounds__(kThreads) void merge_bf16_parts_kernel(const uint16_t* __restrict__ o_parts,
                                                                    const float* __restrict__ lse_parts, int P,
                                                                    int64_t R, int D, uint16_t* __restrict__ out,
                                                                    float* __restrict__ lse_out,
                                                                    const uint16_t* __restrict__ extra_v,
                                                                    int64_t extra_bs, int64_t rows_per_seq) {
  constexpr int NW = kThreads / kWave;
  __shared__ float wsh[NW][1024];
  __shared__ float red[NW - 1][kWave * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = blockIdx.x;
  float* w = wsh[wave];
  // the first round of part loads goes out before the weights, which do not gate them
  const int nd8 = D / 8;
  const bool on = lane < nd8;
  const uint4* base = reinterpret_cast<const uint4*>(o_parts + r * D) + lane;
  const int64_t pstride = R * D / 8;     // uint4 stride between parts
  const uint4* xrow = extra_v ? reinterpret_cast<const uint4*>(extra_v + (r / rows_per_seq) * extra_bs) + lane : nullptr;
  auto part_at = [&](int p) -> uint4 {
    if (!on || p >= P) return make_uint4(0, 0, 0, 0);
    if (xrow && p == P - 1) return *xrow;
    return base[(int64_t)p * pstride];
  };
  uint4 v[kMergePPT];
#pragma unroll
  for (int u = 0; u < kMergePPT; ++u) v[u] = part_at(wave + u * NW);
  float mx = -INFINITY;
  for (int p = lane; p < P; p += kWave) mx = fmaxf(mx, lse_parts[(int64_t)p * R + r]);
  mx = wave_max(mx);
  float tot = 0.f;
  for (int p = lane; p < P; p += kWave) {
    float e = (mx == -INFINITY) ? 0.f : expf(lse_parts[(int64_t)p * R + r] - mx);
    w[p] = e;
    tot += e;
  }
  tot = wave_sum(tot);
  __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int p0 = wave; p0 < P; p0 += NW * kMergePPT) {
    if (p0 != wave) {
#pragma unroll
      for (int u = 0; u < kMergePPT; ++u) v[u] = part_at(p0 + u * NW);
    }
#pragma unroll
    for (int u = 0; u < kMergePPT; ++u) {
      const int p = p0 + u * NW;
      if (p < P) {
        const float wu = w[p];
        const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wu, __uint_as_float(x[e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wu, __uint_as_float(x[e] & 0xffff0000u), acc[2 * e + 1]);
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave - 1][lane * 8 + e] = acc[e];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < NW - 1; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += red[q][lane * 8 + e];
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (on) {
      uint4 o;
      o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      o.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
      o.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
      reinterpret_cast<uint4*>(out + r * D)[lane] = o;
    }
    if (lane == 0 && lse_out) lse_out[r] = (tot > 0.f) ? mx + logf(tot) : -INFINITY;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Dense attention over many queries of a sequence (a prefill chunk) runs two queries per
// workgroup; decode-sized calls keep one query per workgroup.
constexpr int64_t kPairMinQ = 16;
inline bool use_pairs(const AttendArgs& a) { return !a.f32 && !a.f8 && !a.csa && a.D == 512 && a.Q >= kPairMinQ; }

}  // namespace

AttendPlan plan_attend(const AttendArgs& a) {
  AttendPlan p{1, 0, 0};
  const bool pairs = use_pairs(a);
  const int64_t win = a.W < a.L ? a.W : a.L;
  // key list length bound: with pairs, two windows (the union never exceeds both)
  const int64_t n_max = (a.csa ? (int64_t)a.k : a.N) + (win > 0 ? (pairs ? 2 * win : win) : 0);
  if (a.f32 || n_max == 0) {
    p.chunk = (int)(n_max > 0 ? n_max : 1);
    if (a.pool.on) {                      // one (empty) key range and the pooled entry's part
      p.chunk = kTile;
      const int64_t R = a.B * a.Q * a.H;
      p.ws_bytes = align256((size_t)2 * R * a.D * 2) + align256((size_t)2 * R * 4);
    }
    return p;
  }
  const int64_t rows = a.B * (pairs ? (a.Q + 1) / 2 : a.Q);
  int64_t want = (kTargetWorkgroups + rows - 1) / rows;   // about one workgroup per CU
  int64_t max_splits = (n_max + kTile - 1) / kTile;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int64_t chunk = (n_max + want - 1) / want;
  chunk = ((chunk + kTile - 1) / kTile) * kTile;
  if (a.csa && chunk > kMaxCsaChunk) chunk = kMaxCsaChunk;
  if (a.f8 && a.csa && chunk > kListF8) chunk = kListF8;
  int64_t splits = (n_max + chunk - 1) / chunk;
  const int64_t max_splits_m = kMaxSplits - (a.pool.on ? 1 : 0);   // (the pooled HCA entry is a part)
  if (splits > max_splits_m) {            // the merge holds at most kMaxSplits part weights
    chunk = ((n_max + max_splits_m - 1) / max_splits_m + kTile - 1) / kTile * kTile;
    const int64_t cap = a.csa ? (a.f8 ? kListF8 : kMaxCsaChunk) : ((int64_t)1 << 30);
    if (chunk > cap) {
      p.supported = false;
      return p;
    }
    splits = (n_max + chunk - 1) / chunk;
  }
  p.splits = (int)splits;
  p.chunk = (int)chunk;
  const int64_t parts = splits + (a.pool.on ? 1 : 0);         // the pooled HCA entry is one more part
  if (parts > 1) {
    const int64_t R = a.B * a.Q * a.H;
    p.ws_bytes = align256((size_t)parts * R * a.D * 2) + align256((size_t)parts * R * 4);   // bf16 parts
  }
  return p;
}

template <bool kNT>
hipError_t launch_split_kernel(const AttendArgs& a, const AttendPlan& p, dim3 grid, uint16_t* o_part,
                               float* lse_part, hipStream_t st, const PoolLaunch& pl) {
  if (a.f8) {   // D == 512 (checked by the caller)
    DSV4_LAUNCH_MAIN((attend_fp8kv_kernel<512, kNT>), grid, dim3(kThreads * 2), 0, st, a, (int64_t)p.chunk, p.splits,
                     o_part, lse_part);
  } else switch (a.D) {
    case 128: DSV4_LAUNCH_MAIN((attend_bf16_kernel<128, 1, kNT>), grid, dim3(kThreads), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part, pl); break;
    case 256: DSV4_LAUNCH_MAIN((attend_bf16_kernel<256, 1, kNT>), grid, dim3(kThreads), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part, pl); break;
    default: DSV4_LAUNCH_MAIN((attend_bf16_kernel<512, 2, kNT>), grid, dim3(kThreads * 2), 0, st, a, (int64_t)p.chunk, p.splits, o_part, lse_part, pl); break;
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p, void* ws, hipStream_t st) {
  const int64_t rows = a.B * a.Q;
  if (rows == 0) return hipSuccess;
  if (a.f32) {
    size_t smem = (size_t)(a.D + kThreads) * 4;
    DSV4_LAUNCH_MAIN(attend_f32_kernel, dim3((unsigned)a.H, (unsigned)rows), dim3(kThreads), smem, st, a);
    return hipGetLastError();
  }
  uint16_t* o_part = nullptr;
  float* lse_part = nullptr;
  const int64_t R = rows * a.H;
  const int parts = p.splits + (a.pool.on ? 1 : 0);
  if (parts > 1) {
    o_part = reinterpret_cast<uint16_t*>(ws);
    lse_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + align256((size_t)parts * R * a.D * 2));
  }
  if (use_pairs(a)) {
    dim3 pgrid((unsigned)p.splits, (unsigned)(a.B * ((a.Q + 1) / 2)));
    DSV4_LAUNCH_MAIN((attend_bf16_pair_kernel<512>), pgrid, dim3(kThreads * 2), 0, st, a, (int64_t)p.chunk,
                     p.splits, o_part, lse_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(merge_bf16_parts_kernel, dim3((unsigned)R), dim3(kThreads), 0, st, o_part, lse_part, p.splits,
                       R, a.D, reinterpret_cast<uint16_t*>(a.out), a.lse, nullptr, (int64_t)0, (int64_t)1);
    return hipGetLastError();
  }
  // HCA block pooling in the same launch (bf16, D = 512, K|V rows side by side; checked by
  // the caller): cs workgroups per sequence after the attention rows
  PoolLaunch pl;
  if (a.pool.on) {
    pl.grid = a.B * 2;
    pl.rows = (int)rows;
  }
  // one query per sequence: each K/V row is read by one workgroup of the call (streamed)
  const dim3 grid((unsigned)p.splits, (unsigned)(rows + (pl.grid + p.splits - 1) / p.splits));
  hipError_t e = a.Q == 1 ? launch_split_kernel<true>(a, p, grid, o_part, lse_part, st, pl)
                          : launch_split_kernel<false>(a, p, grid, o_part, lse_part, st, pl);
  if (e != hipSuccess || parts == 1) return e;
  // the pooled entry's part: its output is the entry's V row in the cache
  const uint16_t* extra_v = a.pool.on ? reinterpret_cast<const uint16_t*>(a.kc) + a.pool.row * a.kv_rs + a.D : nullptr;
  hipLaunchKernelGGL(merge_bf16_parts_kernel, dim3((unsigned)R), dim3(kThreads), 0, st, o_part, lse_part, parts, R,
                     a.D, reinterpret_cast<uint16_t*>(a.out), a.lse, extra_v, a.kv_bs * a.kv_rs,
                     a.Q * (int64_t)a.H);   // D <= 512: 8 dims per lane
  return hipGetLastError();
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

DSV4_DEBUG_READER(debug_flags_attend)

}  // namespace dsv4
