// moe_kernels.hip -- the fused decode MoE pass for MI355X (gfx950, CDNA4).
//
// One persistent launch: one workgroup of 8 waves per CU, all resident.
//
//   S0  router logits   CU c computes l[r][e] for its experts e = c, c+ncu..
//                       (fp64 sums of exact bf16 products) and sigmoid, and
//                       publishes each score in a slot tagged with the call's
//                       epoch; then raises its flag (epoch + 1).
//   S1  shared up/gate  the shared expert does not depend on routing, so its
//                       8-intermediate tiles are streamed while the other CUs
//                       finish S0.
//   S2  route + group   every CU polls the score slots of every row until
//                       they carry the call's tag, routes every row itself
//                       (no hand-off) and builds the step's group table in
//                       LDS: distinct experts in order of first use, found by
//                       ballot / prefix count, each with its using rows.
//   S3  routed up/gate  jobs (group, 8-intermediate tile) dealt round-robin
//                       over CUs; each job streams 16 weight rows (8 gate + 8
//                       up) once and uses every row of the group as an MFMA
//                       column; SwiGLU mid values go to the workspace.
//   S4  down            after a second flag barrier, CU c owns output rows
//                       [c*hs, (c+1)*hs) and streams that slice of every used
//                       expert's W_down once; per (row, slot) products stay in
//                       LDS.  Unit batches that lie past the step's groups
//                       issue nothing (dead-batch skip).
//   S5  combine         out[r][h] = shared + sum_p w[r][p] * P[r][p][h] in this
//                       row-local order, rounded to bf16 once.
//
// Prior art: sgl-amd-mono-upstream PR #27 (Motivation, Modifications: every
// CTA routes all rows, groups by ballot over the picks, deals 8-intermediate
// up/gate jobs round-robin with every using row as an MFMA column, keeps
// down products in LDS and sums each row in the one-row order; commit 2 skips
// dead down batches); "Daily AI Hotspot 2026-08-21", "Most Worth Your
// Attention Today" (shared L1, routed MMA, shared L2 and fp32 accumulation in
// one persistent kernel that writes bf16 once).
//
// Batch invariance: a column's arithmetic never depends on the batch.  Every
// up/gate and down sum is the same sequence of bf16 MFMAs (column position
// in the tile does not change its bits), the same per-128 block scaling, and
// the same fixed-order reduction over the 8 waves' K ranges; the combine is
// row-local.  Only which CU does the work depends on the batch.
//
// Cross-CU data (scores, mid) is stored at agent scope (written through to
// the device's point of coherence), so raising a flag after it needs only
// the workgroup's own store completion, not an L2 writeback; the one
// exception is the wide stream's mid, stored plainly and published with an
// agent-scope release fence.  Readers poll the flags (or, for scores, the
// epoch tags in the slots themselves) and then acquire at agent scope.
// Each CU owns one flag and raises it by one per phase; a call advances
// every flag by two, so the workspace needs no reset.  Waits are bounded:
// on timeout an error bit is set and the kernel runs on.
#include "moe_internal.h"

#include <atomic>

namespace moe {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kErrScore = 0x1u, kErrMid = 0x2u, kErrTimeout = 0x4u;
constexpr int kSpinLimit = 400000;

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Eight E4M3FN codes (two dwords, k ascending from the low byte) -> bf16x8.
// The conversion is exact (every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

// Eight E2M1 codes (one dword, element k in the low nibble when k is even)
// times a power-of-two block scale -> bf16x8.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  // 2^(c-127); c = 0 gives 2^-127 (a binary32 subnormal), 0xFF is NaN
  if (c == 0xffu) return __uint_as_float(0x7fc00000u);
  if (c == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(c << 23);
}

// This thread's wave in the workgroup, as a scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Loads through global-address-space pointers.  A generic (flat) load also
// counts in the LDS/scalar counter, so every LDS wait would drain it too.
template <class T>
__device__ __forceinline__ T ldg(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return ldg<u32x4>(p); }

// A store other CUs read after a flag barrier: agent scope, written through
// to the device's point of coherence, so that raising the flag needs no
// writeback of this XCD's L2 (see publish).
template <class T>
__device__ __forceinline__ void st_agent(void* a, T v) {
  __hip_atomic_store((__attribute__((address_space(1))) T*)a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a * b for per-lane index arithmetic in the streams, kept apart from a
// following add: fused, the product becomes a 64-bit multiply-add whose
// unused high addend half may share a register with an item in flight, and
// reading it would wait for that load.
__device__ __forceinline__ uint32_t lmul(uint32_t a, uint32_t b) {
  uint32_t t = a * b;
  asm("" : "+v"(t));
  return t;
}

// Optional per-CU phase stamps (build with -DMOE_TIMELINE): thread 0 of each
// workgroup writes s_memrealtime (100 MHz) at phase boundaries into
// p.timeline[blockIdx.x * 64 + i]; MOE_WSTAMP(p, k) has lane 0 of every wave
// write slot 16 + 8k + wave.
#ifdef MOE_TIMELINE
// The stamps are kept in the first 64 LDS words (the layout starts after
// them in such a build) and copied out at the end of the call: a global
// store per stamp would make the compiler wait for it before reusing its
// registers.
extern __shared__ __attribute__((aligned(16))) char moe_tl_smem[];
#define MOE_TL(p, i) (((__attribute__((address_space(3))) uint64_t*)(moe_tl_smem))[i])
#define MOE_STAMP(p, i)                                                                  \
  do {                                                                                   \
    if (threadIdx.x == 0 && (p).timeline) MOE_TL(p, i) = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define MOE_LSTAMP(p, i)                                                                 \
  do {                                                                                   \
    if ((threadIdx.x & 63) == 0 && (p).timeline) MOE_TL(p, i) = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define MOE_WSTAMP(p, k)                                                                 \
  do {                                                                                   \
    if ((threadIdx.x & 63) == 0 && (p).timeline)                                         \
      MOE_TL(p, 16 + 8 * (k) + (threadIdx.x >> 6)) = __builtin_amdgcn_s_memrealtime();  \
  } while (0)
#define MOE_JSTAMP(p, jc)                                                                \
  do {                                                                                   \
    if (threadIdx.x == 0 && (p).timeline && (jc) < 20)                                   \
      MOE_TL(p, 40 + (jc)) = __builtin_amdgcn_s_memrealtime();                           \
  } while (0)
#define MOE_TVAL(p, i, v)                                                                \
  do {                                                                                   \
    if (threadIdx.x == 0 && (p).timeline) MOE_TL(p, i) = (v);                            \
  } while (0)
#else
#define MOE_TVAL(p, i, v) \
  do {                    \
  } while (0)
#define MOE_JSTAMP(p, jc) \
  do {                    \
  } while (0)
#define MOE_STAMP(p, i) \
  do {                  \
  } while (0)
#define MOE_LSTAMP(p, i) \
  do {                   \
  } while (0)
#define MOE_WSTAMP(p, k) \
  do {                   \
  } while (0)
#endif

// ------------------------------------------------------------------ LDS map

struct Lds {
  int32_t* ids;      // [T*K]
  float* w;          // [T*K]
  uint32_t* first;   // [E] first use of each expert
  int32_t* egrp;     // [E] group of each expert
  uint32_t* rmask;   // [E][2] rows using each expert (64-bit mask)
  int32_t* gexp;     // [1+T*K] expert of each group (-1 = shared)
  int32_t* gcnt;     // [1+T*K]
  int32_t* gstart;   // [1+T*K]
  int32_t* cols;     // [T*(K+1)] row*16 + slot
  int32_t* cgrp;     // [T*(K+1)] group of each column
  int32_t* misc;     // [32]: 0 = G, 1 = epoch, 8.. = scan
  uint32_t* ctl;     // [64] chunk-stream counters (see kCtl*)
  float* red;        // [red_slots][red_tiles][kWaves][64][4] job-end partials
  double* rb;        // [kWaves][E] router keys (aliases red and pbuf)
  double* rgs;       // [kWaves][64] group scores
  int32_t* rkept;    // [kWaves][64]
  double* rcb;       // [kWaves][E] top-k candidates: key b
  double* rcs;       // [kWaves][E] and score s
  int32_t* rce;      // [kWaves][E] and expert
  float* pbuf;       // wide: down products [T*(K+1)][hs]; narrow: the per-wave partials (see lds_offsets)
  struct JobDesc* jd;  // narrow: job descriptors (this CU's up/gate jobs, then down jobs)
  uint32_t* wcnt;    // narrow: [kPuWin] chunks of the job in each partial window that have ended
  uint32_t* wgen;    // narrow: [kPuWin] jobs summed out of each window
  uint32_t* ccnt;    // narrow: up/gate chunks claimed by this CU's waves
  uint32_t* cfifo;   // narrow: [kWaves][8] each wave's claimed chunks, fetch side to multiplying side
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// LDS words of the narrow stream's start (misc[]).
constexpr int kMiscNU = 2;      // this CU's up/gate jobs, once routed
constexpr int kMiscReady = 3;   // 1 once the routed jobs' tables are written
constexpr int kMiscRouted = 4;  // rows routed so far (early start)
constexpr int kMiscPolled = 5;  // rows whose scores are in (early start)

// Job-end partials: one 16-column tile per job when a batch has at most 16
// rows (four slots), else four tiles (two slots).
__host__ __device__ inline int red_tiles(int T) { return T > 16 ? kMaxRows / 16 : 1; }
__host__ __device__ inline int red_slots(int T) { return T > 16 ? 2 : 4; }
constexpr size_t kRedTileBytes = 16 * (size_t)kWaves * 64;  // one tile: [wave][lane] f32x4

// Narrow layout (batches of at most 16 rows): every wave keeps its partial
// tiles apart in LDS, and they are summed over the waves in wave order:
//   up/gate  Pu[win][w][col][16], win = local job mod kPuWin (w = 0..7, the
//            job's K-phase; col < T, the job's column; 16 rows: 8 gate then
//            8 up), summed by the wave that ends the job's last chunk
//   down     Pd[kp][row][slot][pitch]  (kp = 0..wpt-1, the K-phase of the
//            waves that share a 16-row down tile; h along the slice),
//            summed in the combine
// Pu and Pd share one region (Pu is done with before Pd is written), which
// also holds the routing scratch before the stream.  The job descriptors
// (qcap up/gate entries, then one down job per group) sit before it.  The wide layout keeps
// job-end partial slots summed by an owner wave, and one copy of the down
// products [row][slot][hs].
constexpr int kPuWin = 8;
struct LdsOffsets {
  size_t ids, w, first, egrp, rmask, gexp, gcnt, gstart, cols, cgrp, misc, ctl, wst, jd, red, pbuf, total;
};
constexpr size_t kJobDescBytes = 48;

__host__ __device__ inline size_t pu_floats(int T) { return (size_t)kPuWin * kWaves * T * 16; }

__host__ __device__ inline LdsOffsets lds_offsets(int T, int K, int E, int hs, int narrow, int wpt, int pitch,
                                                  int qcap) {
  LdsOffsets o;
#ifdef MOE_TIMELINE
  size_t q = 64 * 8;  // the stamps first (see MOE_TL)
#else
  size_t q = 0;
#endif
  const int uses = T * K, gmax = 1 + T * K;
  o.ids = q; q = align_up(q + 4 * (size_t)uses, 16);
  o.w = q; q = align_up(q + 4 * (size_t)uses, 16);
  o.first = q; q = align_up(q + 4 * (size_t)E, 16);
  o.egrp = q; q = align_up(q + 4 * (size_t)E, 16);
  o.rmask = q; q = align_up(q + 8 * (size_t)E, 16);
  o.gexp = q; q = align_up(q + 4 * (size_t)gmax, 16);
  o.gcnt = q; q = align_up(q + 4 * (size_t)gmax, 16);
  o.gstart = q; q = align_up(q + 4 * (size_t)gmax, 16);
  o.cols = q; q = align_up(q + 4 * (size_t)T * (K + 1), 16);
  o.cgrp = q; q = align_up(q + 4 * (size_t)T * (K + 1), 16);
  o.misc = q; q = align_up(q + 4 * 32, 16);
  o.ctl = q; q = align_up(q + 4 * 64, 16);
  o.wst = q; q = align_up(q + 8 * kPuWin + 16 + 4 * kWaves * 8, 16);
  o.jd = q; q = align_up(q + (narrow ? kJobDescBytes * (size_t)(qcap + gmax) : 0), 16);
  // the routing scratch (used before the stream) overlaps the job-end
  // partials and the down products (used in it), except in a narrow call of
  // at most as many rows as waves, whose waves stream while other rows are
  // routed
  o.red = q;
  // routing scratch: rb, rgs, rkept, then the top-k candidates (b, s, e) per wave
  const size_t rs = 8 * (size_t)kWaves * E + 8 * (size_t)kWaves * 64 + 4 * (size_t)kWaves * 64 +
                    20 * (size_t)kWaves * E;
  size_t end;
  if (narrow) {
    const size_t pu = 4 * pu_floats(T);
    const size_t pd = 4 * (size_t)wpt * T * (K + 1) * pitch;
    const size_t need = pu > pd ? pu : pd;
    if (T <= kWaves) {
      o.pbuf = align_up(q + rs, 16);
      end = o.pbuf + need;
    } else {
      o.pbuf = q;
      end = q + (need > rs ? need : rs);
    }
  } else {
    const size_t rd = (size_t)red_slots(T) * red_tiles(T) * kRedTileBytes;
    const size_t need = rd + 4 * (size_t)T * (K + 1) * hs;
    o.pbuf = q + rd;
    end = q + (need > rs ? need : rs);
  }
  o.total = align_up(end, 16);
  return o;
}

#ifndef MOE_RES_WIDE_TU
size_t stream_geometry(Params& p, int narrow) {
  const int nrt = (p.hs + 15) / 16;
  p.nrt_p = nrt <= 1 ? 1 : nrt <= 2 ? 2 : 4;
  p.wpt = kWaves / p.nrt_p;
  p.pitch = 16 * nrt;
  p.narrow = narrow;
  // up/gate job entries: a CU's share of the largest job count the batch
  // can have
  const int gmax = 1 + (p.E < p.T * p.K ? p.E : p.T * p.K);
  const int sh_tiles = p.n_shared ? p.Is / 8 : 0;
  const long jobs = sh_tiles + (long)(gmax - 1) * (p.I / 8);
  p.qcap = (int)((jobs + p.ncu - 1) / p.ncu);
  return lds_offsets(p.T, p.K, p.E, p.hs, p.narrow, p.wpt, p.pitch, p.qcap).total;
}
#endif

__device__ inline Lds lds_map(char* base, const Params& p) {
  LdsOffsets o = lds_offsets(p.T, p.K, p.E, p.hs, p.narrow, p.wpt, p.pitch, p.qcap);
  Lds L;
  L.ids = (int32_t*)(base + o.ids);
  L.w = (float*)(base + o.w);
  L.first = (uint32_t*)(base + o.first);
  L.egrp = (int32_t*)(base + o.egrp);
  L.rmask = (uint32_t*)(base + o.rmask);
  L.gexp = (int32_t*)(base + o.gexp);
  L.gcnt = (int32_t*)(base + o.gcnt);
  L.gstart = (int32_t*)(base + o.gstart);
  L.cols = (int32_t*)(base + o.cols);
  L.cgrp = (int32_t*)(base + o.cgrp);
  L.misc = (int32_t*)(base + o.misc);
  L.ctl = (uint32_t*)(base + o.ctl);
  L.jd = (JobDesc*)(base + o.jd);
  L.wcnt = (uint32_t*)(base + o.wst);
  L.wgen = L.wcnt + kPuWin;
  L.ccnt = L.wgen + kPuWin;
  L.cfifo = L.ccnt + 4;
  L.red = (float*)(base + o.red);
  L.pbuf = (float*)(base + o.pbuf);
  L.rb = (double*)(base + o.red);
  L.rgs = L.rb + (size_t)kWaves * p.E;
  L.rkept = (int32_t*)(L.rgs + (size_t)kWaves * 64);
  L.rcb = (double*)(L.rkept + (size_t)kWaves * 64);
  L.rcs = L.rcb + (size_t)kWaves * p.E;
  L.rce = (int32_t*)(L.rcs + (size_t)kWaves * p.E);
  return L;
}

// ------------------------------------------------------------------ flags

// Raise this CU's flag to `value` after the workgroup's prior stores that
// other CUs read.  Those stores are agent-scope (st_agent), so once each
// wave has waited for its own stores to complete they are visible device
// wide: the workgroup meets and one thread stores the flag, with no
// writeback of the L2 (an agent-scope release fence would write back the
// whole XCD's L2, and with every CU of an XCD doing so at once that costs
// microseconds).
__device__ inline void publish(const Params& p, uint32_t value) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(&p.flags[blockIdx.x], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave polls every CU's flag until all have reached `target`
// (wrap-around safe), then acquires at agent scope.
__device__ inline void poll_flags(const Params& p, uint32_t target) {
  const int lane = threadIdx.x & 63;
  int spins = 0;
  for (;;) {
    bool ok = true;
    for (int i = lane; i < p.ncu; i += 64) {
      uint32_t v = __hip_atomic_load(&p.flags[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = ok && ((int32_t)(v - target) >= 0);
    }
    if (__all(ok)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) set_err(p.err, kErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Wait until every CU's flag has reached `target`: wave 0 polls and
// acquires, the workgroup barrier orders the rest.
__device__ inline void wait_all(const Params& p, uint32_t target) {
  if (threadIdx.x < 64) poll_flags(p, target);
  __syncthreads();
}

// ------------------------------------------------------------------ S0 logits

// Score slots: s[r][e] as two 64-bit words (tag, high half of s) and (tag,
// low half of s), each stored at agent scope; tag = the call's epoch + 1,
// so a reader polls the slots themselves and needs no flag barrier (a slot
// is current once both its words carry the call's tag).  The key
// b = s + bias is recomputed by the reader in the same fp64 operation.
__device__ __forceinline__ void publish_score(const Params& p, int r, int e, double s, uint32_t tag) {
  uint64_t* dst = (uint64_t*)p.scores + ((size_t)r * p.E + e) * 2;
  const uint64_t sb = __builtin_bit_cast(uint64_t, s);
  st_agent<uint64_t>(dst, ((uint64_t)tag << 32) | (sb >> 32));
  st_agent<uint64_t>(dst + 1, ((uint64_t)tag << 32) | (sb & 0xffffffffull));
}

__device__ inline double load_bias(const Params& p, int e) {
  if (p.bias_bf16) return (double)bf16_bits_to_f32(((const uint16_t*)p.bias)[e]);
  return (double)((const float*)p.bias)[e];
}

// The same in two steps: the bits (bf16 or f32), then the value.
__device__ __forceinline__ uint32_t load_bias_raw(const Params& p, int e) {
  return p.bias_bf16 ? (uint32_t)((const uint16_t*)p.bias)[e] : ((const uint32_t*)p.bias)[e];
}
__device__ __forceinline__ double bias_from_raw(const Params& p, uint32_t raw) {
  return (double)(p.bias_bf16 ? bf16_bits_to_f32(raw) : __builtin_bit_cast(float, raw));
}

// ------------------------------------------------------------------ S2 routing

__device__ __forceinline__ bool key_before(double b1, int e1, double b2, int e2) {
  return b1 > b2 || (b1 == b2 && e1 < e2);
}

// Cross-lane moves that need no LDS round trip: DPP within 16-lane rows
// (xor 1, xor 2, half-row mirror, row mirror) and a swizzle (xor 16 within
// 32 lanes).  After the four DPP steps of an all-reduce every lane holds its
// row's result; after the swizzle, its 32-lane half's.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ int xlane(int v) {
  if (CTRL == kSwizzleXor16) return __builtin_amdgcn_ds_swizzle(v, kSwizzleXor16);
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double xlane_d(double v) {
  const long long u = __double_as_longlong(v);
  const int lo = xlane<CTRL>((int)(u & 0xffffffffll)), hi = xlane<CTRL>((int)(u >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// (key, index) maximum under key_before, one exchange step.
template <int CTRL>
__device__ __forceinline__ void best_step(double& b, int& e) {
  const double ob = xlane_d<CTRL>(b);
  const int oe = xlane<CTRL>(e);
  if (key_before(ob, oe, b, e)) {
    b = ob;
    e = oe;
  }
}
// The wave's best (key, index); the result is the same in every lane.
__device__ __forceinline__ void wave_best(double& b, int& e) {
  best_step<kDppXor1>(b, e);
  best_step<kDppXor2>(b, e);
  best_step<kDppHalfMirror>(b, e);
  best_step<kDppMirror>(b, e);
  best_step<kSwizzleXor16>(b, e);
  const double b0 = readlane_d(b, 0), b1 = readlane_d(b, 32);
  const int e0 = __builtin_amdgcn_readlane(e, 0), e1 = __builtin_amdgcn_readlane(e, 32);
  const bool second = key_before(b1, e1, b0, e0);
  b = second ? b1 : b0;
  e = second ? e1 : e0;
}

// Unsigned maximum over the wave (every lane gets it).
template <int CTRL>
__device__ __forceinline__ uint32_t umax_step(uint32_t v) {
  const uint32_t o = (uint32_t)xlane<CTRL>((int)v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = umax_step<kDppXor1>(v);
  v = umax_step<kDppXor2>(v);
  v = umax_step<kDppHalfMirror>(v);
  v = umax_step<kDppMirror>(v);
  v = umax_step<kSwizzleXor16>(v);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  return a > b ? a : b;
}

// Order-preserving 32-bit code of a float (larger float, larger code);
// every code of a float is above 0, which marks "no candidate".
__device__ __forceinline__ uint32_t ord32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum over the wave in a fixed tree (the result is the same in every lane:
// each step adds two equal-shaped partial sums, and fp addition commutes).
__device__ __forceinline__ double wave_sum_d(double v) {
  v += xlane_d<kDppXor1>(v);
  v += xlane_d<kDppXor2>(v);
  v += xlane_d<kDppHalfMirror>(v);
  v += xlane_d<kDppMirror>(v);
  v += xlane_d<kSwizzleXor16>(v);
  return readlane_d(v, 0) + readlane_d(v, 32);
}

// l[r][e] = sum_h x[r][h] * Wr[e][h] for this CU's experts e = c, c+ncu, ..
// and every row, in fp64 (bf16 products are exact).  Each dot is split into
// 8 contiguous chunks of H/8, one per wave; lane l sums the 16-byte groups l
// and l+64 of its chunk in order, the lanes are summed by a fixed tree and
// the chunk sums in wave order.  Up to 4 dots' loads are issued before any
// is summed.  Then s = sigmoid(l) and b = s + bias go to the workspace.
__device__ inline void router_logits(const Params& p, const Lds& L, uint32_t epoch, uint32_t dtag) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int ch = p.H / kWaves, ngrp = ch >> 3;
  const int g0 = lane < ngrp ? lane : ngrp - 1, g1 = lane + 64 < ngrp ? lane + 64 : g0;
  const int nexp = p.E > (int)blockIdx.x ? (p.E - 1 - (int)blockIdx.x) / p.ncu + 1 : 0;
  const int nd = nexp * p.T;
  double* part = L.rb;  // [dot][wave]
  // the bias bits of this thread's first dot, loaded ahead of the sums
  const int d_first = threadIdx.x;
  uint32_t braw = d_first < nd ? load_bias_raw(p, (int)blockIdx.x + (d_first / p.T) * p.ncu) : 0u;
  // four dots per pass; the first pass is peeled so that no loop-entry
  // wait (for the previous pass's unused loads) holds its loads back
  auto pass = [&](int d0) {
    u32x4 xv[4][2], wv[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = d0 + j < nd ? d0 + j : nd - 1;
      const int e = (int)blockIdx.x + (d / p.T) * p.ncu, r = d % p.T;
      const uint16_t* xr = p.x + (size_t)r * p.H + (size_t)wave * ch;
      const uint16_t* wr = p.router_w + (size_t)e * p.H + (size_t)wave * ch;
      xv[j][0] = ld16(xr + 8 * g0);
      wv[j][0] = ld16(wr + 8 * g0);
      xv[j][1] = ld16(xr + 8 * g1);
      wv[j][1] = ld16(wr + 8 * g1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (d0 + j < nd) {
        double acc = 0.0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (q == 0 ? lane < ngrp : lane + 64 < ngrp) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t xa = xv[j][q][i], wa = wv[j][q][i];
              acc = fma((double)bf16_bits_to_f32(xa & 0xffffu), (double)bf16_bits_to_f32(wa & 0xffffu), acc);
              acc = fma((double)bf16_bits_to_f32(xa >> 16), (double)bf16_bits_to_f32(wa >> 16), acc);
            }
          }
        }
        acc = wave_sum_d(acc);
        if (lane == 0) part[(d0 + j) * kWaves + wave] = acc;
      }
      __builtin_amdgcn_sched_barrier(0);  // one dot's conversions at a time
    }
  };
  if (nd > 0) pass(0);
  for (int d0 = 4; d0 < nd; d0 += 4) pass(d0);
  __syncthreads();
  asm volatile("" : "+v"(epoch), "+v"(braw));  // first read here, after the router loads
  for (int d = threadIdx.x; d < nd; d += kThreads) {
    double l = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += part[d * kWaves + w];
    const int e = (int)blockIdx.x + (d / p.T) * p.ncu, r = d % p.T;
    const double s = 1.0 / (1.0 + exp(-l));
    const double b = s + (d == d_first ? bias_from_raw(p, braw) : load_bias(p, e));
    if (!isfinite(l) || !isfinite(b)) set_err(p.err, kErrScore);
    publish_score(p, r, e, s, epoch + dtag);
  }
}

// The same logits with one wave per (row, expert), in the same summation
// order as router_logits, so that a logit has the same bits whatever the
// batch size (the two forms are chosen by batch size): the wave walks the 8
// chunks of H/8 in order, lane l sums the 16-byte groups l and l+64 of a
// chunk (8 elements each, in order), the lanes are summed by the same fixed
// tree (wave_sum_d), and the chunk sums are added in chunk order.  The
// loads of NC chunks are issued before their products are summed (all 8
// with LATE).  Used from 8 rows up, where every wave has rows of its own.
// LATE: `v` is the epoch, a load still in flight, first read once the sums
// are formed (tag = epoch + 1); otherwise `v` is the tag.
template <bool LATE>
__device__ inline void router_logits_rows(const Params& p, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= kWaves) return;
  const int ch = p.H / kWaves, ngrp = ch >> 3;
  const int g0 = lane < ngrp ? lane : ngrp - 1, g1 = lane + 64 < ngrp ? lane + 64 : g0;
  constexpr int NC = LATE ? kWaves : kWaves / 2;
  for (int e = blockIdx.x; e < p.E; e += p.ncu) {
    const uint16_t* wr = p.router_w + (size_t)e * p.H;
    // LATE: the bias bits are converted once the sums are formed
    const uint32_t braw = LATE ? load_bias_raw(p, e) : 0u;
    const double bias = LATE ? 0.0 : load_bias(p, e);
    for (int r = wave; r < p.T; r += kWaves) {
      const uint16_t* xr = p.x + (size_t)r * p.H;
      double l = 0.0;
      for (int c0 = 0; c0 < kWaves; c0 += NC) {
        u32x4 xv[NC][2], wv[NC][2];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const size_t o = (size_t)(c0 + c) * ch;
          xv[c][0] = ld16(xr + o + 8 * g0);
          wv[c][0] = ld16(wr + o + 8 * g0);
          xv[c][1] = ld16(xr + o + 8 * g1);
          wv[c][1] = ld16(wr + o + 8 * g1);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          double acc = 0.0;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (q == 0 ? lane < ngrp : lane + 64 < ngrp) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t xa = xv[c][q][i], wa = wv[c][q][i];
                acc = fma((double)bf16_bits_to_f32(xa & 0xffffu), (double)bf16_bits_to_f32(wa & 0xffffu), acc);
                acc = fma((double)bf16_bits_to_f32(xa >> 16), (double)bf16_bits_to_f32(wa >> 16), acc);
              }
            }
          }
          l += wave_sum_d(acc);
        }
      }
      uint32_t ep = v, br = braw;
      if (LATE) asm volatile("" : "+v"(ep), "+v"(br));
      if (lane == 0) {
        double s = 1.0 / (1.0 + exp(-l));
        double b = s + (LATE ? bias_from_raw(p, br) : bias);
        if (!isfinite(l) || !isfinite(b)) set_err(p.err, kErrScore);
        publish_score(p, r, e, s, LATE ? ep + 1 : v);
      }
    }
  }
}

// Two largest values (t1 >= t2) of an aligned lane group, one exchange step.
template <int CTRL>
__device__ __forceinline__ void top2_step(double (&t1)[4], double (&t2)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double o1 = xlane_d<CTRL>(t1[i]), o2 = xlane_d<CTRL>(t2[i]);
    const double hi = fmax(t1[i], o1), lo = fmin(t1[i], o1);
    t2[i] = fmax(lo, fmax(t2[i], o2));
    t1[i] = hi;
  }
}

__device__ __forceinline__ double pick4(const double (&v)[4], int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// Routes row r with one wave: group stage (sum of the two best keys per
// group, keep k_g groups by (score desc, index asc)), then K rounds of wave
// argmax over (key desc, index asc); weights s/sum(s)*scale in fp64.
// Lane l holds experts l, l+64, l+128, l+192.
// POLL: poll row r's score slots (agent-scope loads) until every one
// carries this call's tag (bounded: on timeout the error bit is set and
// routing runs on).  Otherwise the flags have been waited for and the slots
// are read once with plain loads (many rows per wave: they hit in L2).
template <bool POLL>
__device__ inline void route_row(const Params& p, const Lds& L, int r, uint32_t tag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  typedef __attribute__((address_space(1))) uint64_t G64;
  const G64* sc = (const G64*)p.scores + (size_t)r * p.E * 2;
  uint64_t w0[4] = {0, 0, 0, 0}, w1[4] = {0, 0, 0, 0};
  double bias[4];  // loaded first: they do not depend on the scores
#pragma unroll
  for (int i = 0; i < 4; ++i) bias[i] = lane + 64 * i < p.E ? load_bias(p, lane + 64 * i) : 0.0;
  if (!POLL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < p.E) {
        w0[i] = sc[2 * e];
        w1[i] = sc[2 * e + 1];
      }
    }
  }
  for (int spins = 0; POLL;) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < p.E) {
        w0[i] = __hip_atomic_load(sc + 2 * e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w1[i] = __hip_atomic_load(sc + 2 * e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = ready && (uint32_t)(w0[i] >> 32) == tag && (uint32_t)(w1[i] >> 32) == tag;
      }
    }
    if (__all(ready)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) set_err(p.err, kErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (r == 0) MOE_LSTAMP(p, 9);
  if (POLL && lane == 0)  // rows whose scores are in (see narrow_forward)
    __hip_atomic_fetch_add((__attribute__((address_space(3))) uint32_t*)(L.misc + kMiscPolled), 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  double bv[4], sv[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    alive[i] = e < p.E;
    const double s = __builtin_bit_cast(double, (w0[i] << 32) | (w1[i] & 0xffffffffull));
    const double b = alive[i] ? s + bias[i] : -INFINITY;
    sv[i] = alive[i] ? s : 0.0;
    bv[i] = isnan(b) ? -INFINITY : b;
  }
  if (r == 0) MOE_LSTAMP(p, 60);
  if (p.ng > 1) {
    const int gsz = p.E / p.ng;
    if (gsz <= 64 && (gsz & (gsz - 1)) == 0) {
      // each group is an aligned run of gsz lanes of one slot: butterfly
      double t1[4], t2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t1[i] = bv[i];
        t2[i] = -INFINITY;
      }
      if (gsz > 1) top2_step<kDppXor1>(t1, t2);
      if (gsz > 2) top2_step<kDppXor2>(t1, t2);
      if (gsz > 4) top2_step<kDppHalfMirror>(t1, t2);
      if (gsz > 8) top2_step<kDppMirror>(t1, t2);
      if (gsz > 16) top2_step<kSwizzleXor16>(t1, t2);
      if (gsz > 32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double o1 = __shfl_xor(t1[i], 32, 64), o2 = __shfl_xor(t2[i], 32, 64);
          const double hi = fmax(t1[i], o1), lo = fmin(t1[i], o1);
          t2[i] = fmax(lo, fmax(t2[i], o2));
          t1[i] = hi;
        }
      }
      double gs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = t1[i] + t2[i];
      // rank of this lane's group j_i = (lane + 64 i) / gsz among all groups
      if (POLL && gsz == 32) {
        // groups 2i and 2i+1 are the halves of slot i: a swap of halves
        // gives every lane both scores, so every lane holds all groups
        double glo[4], ghi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long u = __double_as_longlong(gs[i]);
          const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
          const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
          glo[i] = __longlong_as_double(((long long)hi[0] << 32) | lo[0]);
          ghi[i] = __longlong_as_double(((long long)hi[1] << 32) | lo[1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int own = 2 * i + (lane >> 5);
          int rank = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < p.ng) rank += key_before((j & 1) ? ghi[j >> 1] : glo[j >> 1], j, gs[i], own) ? 1 : 0;
          alive[i] = alive[i] && rank < p.kg;
        }
      } else {
        int rank[4] = {0, 0, 0, 0};
        for (int j = 0; j < p.ng; ++j) {
          const int first = j * gsz;
          const double gj = readlane_d(pick4(gs, first >> 6), first & 63);
#pragma unroll
          for (int i = 0; i < 4; ++i) rank[i] += key_before(gj, j, gs[i], (lane + 64 * i) / gsz) ? 1 : 0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) alive[i] = alive[i] && rank[i] < p.kg;
      }
    } else {
      double* rb = L.rb + (size_t)wave * p.E;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (alive[i]) rb[lane + 64 * i] = bv[i];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < p.ng) {
        double t1 = -INFINITY, t2 = -INFINITY;
        for (int e = lane * gsz; e < (lane + 1) * gsz; ++e) {
          double v = rb[e];
          if (v > t1) { t2 = t1; t1 = v; }
          else if (v > t2) { t2 = v; }
        }
        L.rgs[wave * 64 + lane] = t1 + t2;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < p.ng) {
        const double mine = L.rgs[wave * 64 + lane];
        int rank = 0;
        for (int j = 0; j < p.ng; ++j) rank += key_before(L.rgs[wave * 64 + j], j, mine, lane) ? 1 : 0;
        L.rkept[wave * 64 + lane] = rank < p.kg;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (alive[i]) alive[i] = L.rkept[wave * 64 + (lane + 64 * i) / gsz] != 0;
    }
  }
  if (r == 0) MOE_LSTAMP(p, 14);
  // Top-k among the alive experts by (b desc, e asc), in two steps.
  // (1) Rounded to fp32, keys keep their order (ties aside), so the k-th
  // largest rounded key t is the rounding of the k-th largest exact key,
  // and every expert whose rounded key is >= t holds all k winners.  t is
  // found by rounds of wave maximum, each retiring every key equal to it.
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = alive[i] ? ord32((float)bv[i]) : 0u;
  uint32_t t = 0u;
  for (int cnt = 0; cnt < p.K;) {
    uint32_t m = key[0] > key[1] ? key[0] : key[1];
    m = m > key[2] ? m : key[2];
    m = m > key[3] ? m : key[3];
    t = wave_umax(m);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool eq = key[i] == t;
      cnt += __popcll(__ballot(eq));
      if (eq) key[i] = 0u;
    }
    if (t == 0u) break;  // fewer alive experts than k (not reachable with validated shapes)
  }
  // (2) The candidates go to LDS in expert order; each is ranked exactly
  // by (b desc, e asc) against all of them.
  double* cb = L.rcb + (size_t)wave * p.E;
  double* cs = L.rcs + (size_t)wave * p.E;
  int32_t* ce = L.rce + (size_t)wave * p.E;
  int nc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool c = alive[i] && ord32((float)bv[i]) >= t;
    const unsigned long long bal = __ballot(c);
    if (c) {
      const int pos = nc + __popcll(bal & ((1ull << lane) - 1ull));
      cb[pos] = bv[i];
      cs[pos] = sv[i];
      ce[pos] = lane + 64 * i;
    }
    nc += __popcll(bal);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  double* ps = L.rgs + (size_t)wave * 64;  // the winners' s in pick order
  if (POLL && nc <= 8) {
    // lane 8a + c compares candidate c with candidate a; a's rank is the
    // count of its lane group's bits
    const int a = lane >> 3, c = lane & 7;
    const bool in = a < nc && c < nc;
    const int ia = in ? a : 0, ic = in ? c : 0;
    const double ba = cb[ia], bc = cb[ic];
    const int ea = ce[ia], ec = ce[ic];
    const double sa = cs[ia];
    const unsigned long long before = __ballot(in && key_before(bc, ec, ba, ea));
    const int rank = __popc((uint32_t)(before >> (8 * a)) & 0xffu);
    if (in && c == 0 && rank < p.K) {
      L.ids[r * p.K + rank] = ea;
      ps[rank] = sa;
    }
  } else {
    for (int j = lane; j < nc; j += 64) {
      const double bj = cb[j];
      const int ej = ce[j];
      int rank = 0;
      for (int q = 0; q < nc; ++q) rank += key_before(cb[q], ce[q], bj, ej) ? 1 : 0;
      if (rank < p.K) {
        L.ids[r * p.K + rank] = ej;
        ps[rank] = cs[j];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (r == 0) MOE_LSTAMP(p, 15);
  if (POLL) {
    // every lane forms the same sum in pick order; lane k writes weight k
    double ssum = 0.0;
    for (int k = 0; k < p.K; ++k) ssum += ps[k];
    if (lane < p.K) L.w[r * p.K + lane] = (float)(ps[lane] / ssum * p.routed_scale);
  } else if (lane == 0) {  // (the same values; this form keeps the wide stream's code as measured)
    double ssum = 0.0;
    for (int k = 0; k < p.K; ++k) ssum += ps[k];
    for (int k = 0; k < p.K; ++k) L.w[r * p.K + k] = (float)(ps[k] / ssum * p.routed_scale);
  }
}

// ------------------------------------------------------------------ S2 grouping

// Distinct experts of the step in order of first use over u = r*K + slot
// (group 0 = shared expert when present), each group's columns in ascending
// u.  Needs L.ids; whole workgroup; ends synchronised.
// Orders this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// gstart[g] = base + sum of gcnt over groups g0..g-1, for g0 <= g < G, by
// one wave (64 groups per pass).
__device__ inline void scan_gstart(const Lds& L, int g0, int G, int base) {
  const int lane = threadIdx.x & 63;
  for (int c0 = g0; c0 < G; c0 += 64) {
    const int g = c0 + lane;
    const int c = g < G ? L.gcnt[g] : 0;
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (g < G) L.gstart[g] = base + v - c;
    base += __shfl(v, 63, 64);
  }
}

// Column of use u = r*K + slot within its group: the rows using an expert,
// in ascending order (a row picks an expert at most once).
__device__ __forceinline__ int use_rank(const Lds& L, int e, int r) {
  const uint32_t lo = L.rmask[2 * e], hi = L.rmask[2 * e + 1];
  return r < 32 ? __popc(lo & ((1u << r) - 1u)) : __popc(lo) + __popc(hi & ((1u << (r - 32)) - 1u));
}

// The grouping of up to 64 uses by one wave (the narrow stream's wave 7),
// one use per lane, no workgroup barriers.
__device__ inline void groups_one_wave(const Params& p, const Lds& L) {
  const int lane = threadIdx.x & 63;
  const int U = p.T * p.K;
  {
    {
      const bool valid = lane < U;
      const int e = valid ? L.ids[lane] : 0, r = lane / p.K;
      if (valid) {
        L.first[e] = 0xffffffffu;
        L.rmask[2 * e] = 0u;
        L.rmask[2 * e + 1] = 0u;
      }
      wave_sync();
      if (valid) {
        atomicMin(&L.first[e], (uint32_t)lane);
        atomicOr(&L.rmask[2 * e + (r >> 5)], 1u << (r & 31));
      }
      wave_sync();
      const bool isf = valid && L.first[e] == (uint32_t)lane;
      const unsigned long long m = __ballot(isf);
      const int G = p.n_shared + __popcll(m);
      if (isf) {
        const int g = p.n_shared + __popcll(m & ((1ull << lane) - 1ull));
        L.egrp[e] = g;
        L.gexp[g] = e;
        L.gcnt[g] = __popc(L.rmask[2 * e]) + __popc(L.rmask[2 * e + 1]);
      }
      if (lane == 0) {
        L.misc[0] = G;
        if (p.n_shared) {
          L.gexp[0] = -1;
          L.gcnt[0] = p.T;
          L.gstart[0] = 0;
        }
      }
      wave_sync();
      scan_gstart(L, p.n_shared, G, p.n_shared ? p.T : 0);
      wave_sync();
      if (p.n_shared && lane < p.T) {
        L.cols[lane] = lane * 16 + p.K;
        L.cgrp[lane] = 0;
      }
      if (valid) {
        const int g = L.egrp[e], c = L.gstart[g] + use_rank(L, e, r);
        L.cols[c] = r * 16 + (lane - r * p.K);
        L.cgrp[c] = g;
      }
    }
  }
}

__device__ inline void build_groups(const Params& p, const Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = p.T * p.K;
  if (U <= 64) {
    if (wave == 0) groups_one_wave(p, L);
    __syncthreads();
    return;
  }
  for (int e = tid; e < p.E; e += kThreads) {
    L.first[e] = 0xffffffffu;
    L.rmask[2 * e] = 0u;
    L.rmask[2 * e + 1] = 0u;
  }
  __syncthreads();
  for (int u = tid; u < U; u += kThreads) {
    const int e = L.ids[u], r = u / p.K;
    atomicMin(&L.first[e], (uint32_t)u);
    atomicOr(&L.rmask[2 * e + (r >> 5)], 1u << (r & 31));
  }
  __syncthreads();
  // exclusive prefix count of first uses, 512 uses per pass
  int base = p.n_shared;
  for (int u0 = 0; u0 < U; u0 += kThreads) {
    const int u = u0 + tid;
    const bool isf = u < U && L.first[L.ids[u]] == (uint32_t)u;
    const unsigned long long m = __ballot(isf);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) L.misc[8 + wave] = __popcll(m);
    __syncthreads();
    int wbase = base;
    for (int w = 0; w < wave; ++w) wbase += L.misc[8 + w];
    int total = 0;
    for (int w = 0; w < kAllWaves; ++w) total += L.misc[8 + w];
    if (isf) {
      const int g = wbase + before;
      const int e = L.ids[u];
      L.egrp[e] = g;
      L.gexp[g] = e;
      L.gcnt[g] = __popc(L.rmask[2 * e]) + __popc(L.rmask[2 * e + 1]);
    }
    base += total;
    __syncthreads();
  }
  const int G = base;
  if (wave == 0) {
    if (lane == 0) {
      L.misc[0] = G;
      if (p.n_shared) {
        L.gexp[0] = -1;
        L.gcnt[0] = p.T;
        L.gstart[0] = 0;
      }
    }
    scan_gstart(L, p.n_shared, G, p.n_shared ? p.T : 0);
  }
  __syncthreads();
  if (p.n_shared)
    for (int r = tid; r < p.T; r += kThreads) {
      L.cols[r] = r * 16 + p.K;
      L.cgrp[r] = 0;
    }
  for (int u = tid; u < U; u += kThreads) {
    const int e = L.ids[u], r = u / p.K, slot = u - r * p.K;
    const int g = L.egrp[e], c = L.gstart[g] + use_rank(L, e, r);
    L.cols[c] = r * 16 + slot;
    L.cgrp[c] = g;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ weight stream
//
// Each CU walks a sequence of jobs: its shared-expert up/gate tiles, its
// routed up/gate tiles (16 weight rows, 8 gate + 8 up, over all of H), then
// its 16-row down tiles of every used expert (over that expert's
// intermediate size).  The 8 waves split every job along the reduction
// axis: wave w owns the 128-element K-blocks w, w+8, w+16, ...  One such
// K-block of one job is an item: the 16 rows' weights (FP8 32 bytes or
// MXFP4 16 bytes per lane), the activations of the group's columns and the
// block scale.  A wave loads its items straight from HBM into registers,
// D items ahead of the one it multiplies; every item issues the same number
// of loads, so the in-order wait for item n leaves items n+1..n+D-1 in
// flight.  (An LDS ring fed by LDS-DMA reached a lower and less steady
// share of HBM bandwidth.)


// Wave-uniform loop state, re-asserted as uniform: the compiler's uniformity
// analysis loses track of it across the stream loops (asm results, loop
// exits) and then keeps it in vector registers behind masked branches.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A kernel-argument pointer taken through readfirstlane.  Choosing between
// two fields of the argument block is otherwise folded into one load from a
// chosen address, which forces the whole block into scratch memory.
template <class T>
__device__ __forceinline__ T* arg_ptr(T* q) {
  const uint64_t v = (uint64_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// LDS accesses of the stream's synchronisation go through these.  Reads
// wait for themselves; stores are not waited for (a wave's LDS operations
// complete in order, so a later flag store is seen after the data it
// publishes, and a compiler-placed lgkmcnt wait that follows stays
// sufficient: an extra older operation completes first).
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}
template <class P>
__device__ __forceinline__ uint32_t lds_ld32(P p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return v;
}
// For an address every lane of the wave shares.
__device__ __forceinline__ int lds_ldi_uniform(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane((int)lds_ld32(p));
}
__device__ __forceinline__ void lds_st32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st128(void* p, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}

// Stream counters in LDS.  Every counter counts up from 0 within a launch
// and is written by one wave only.
constexpr int kCtlProg = 0;    // [8]  jobs wave w has ended
constexpr int kCtlPart = 16;   // [8]  jobs whose partials wave w has stored
constexpr int kCtlSlot = 24;   // [4]  1 + the last job summed out of partial slot s
constexpr int kCtlMidOut = 40; // [8]  1 once wave w's mid stores are complete
constexpr int kCtlCrossed = 48;// [1]  1 once wave 0 has seen every CU's mid

// Minimum of N consecutive LDS counters (N = 1 or 8), one round trip.  Every
// lane reads the same words; the result goes through readfirstlane so the
// compiler knows it is uniform.
template <int N>
__device__ __forceinline__ uint32_t lds_min(const uint32_t* a) {
  if (N == 1) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(a)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
  } else {
    u32x4 a0, a1;
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a0), "=&v"(a1) : "v"(lds_off(a)) : "memory");
    uint32_t m = a0[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) m = a0[i] < m ? a0[i] : m;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = a1[i] < m ? a1[i] : m;
    return __builtin_amdgcn_readfirstlane(m);
  }
}

// Spins until the minimum of N counters reaches `target`.  Bounded: on
// timeout the error bit is set and `ok` latches false, after which every
// wait of this wave returns at once (the kernel then finishes with wrong
// values, never hangs).
template <int N>
__device__ inline uint32_t lds_wait(const Params& p, const uint32_t* a, uint32_t target, bool& ok) {
  if (!ok) return target;
  int spins = 0;
  uint32_t v;
  while ((v = lds_min<N>(a)) < target) {
    if (++spins > kSpinLimit) {
      set_err(p.err, kErrTimeout);
      ok = false;
      return target;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return v;
}

// Column tiles a group can have: 1 when NPRE is 1 (batches of at most 16
// rows), else up to 4 (64 rows).
template <int NPRE>
constexpr int max_tiles() { return NPRE == 1 ? 1 : kMaxRows / 16; }
// Items in flight per wave.
template <int NPRE>
constexpr int depth() { return NPRE == 1 ? 5 : 3; }

struct Sched {
  int sh_tiles;  // shared up/gate jobs (I_s / 8)
  int rt_tiles;  // routed up/gate jobs per group (I / 8)
  int n_jobs;    // all up/gate jobs, known after routing
  int G;         // groups, known after routing
  int h0, hc;    // this CU's down rows
  int nrt;       // 16-row tiles of them
  int nrt_p, wpt;  // tiles rounded up to 1, 2 or 4; waves per tile
  int narrow;    // each wave walks only its own down tile's jobs
};

// Position in this CU's job sequence.
struct It {
  int phase;  // 0 shared up/gate, 1 routed up/gate, 2 down, 3 end
  int j;      // up/gate: global job index; down: group
  int rt;     // down: 16-row tile of this CU's slice
  int g;      // the job's group (kept current by settle / next_job)
  int tile;   // up/gate: its 8-intermediate tile of that group
};

__device__ __forceinline__ void uni(It& c) {
  c.phase = uni(c.phase);
  c.j = uni(c.j);
  c.rt = uni(c.rt);
  c.g = uni(c.g);
  c.tile = uni(c.tile);
}

// Smallest j >= begin with j = blockIdx.x (mod ncu): jobs are dealt round-robin.
__device__ __forceinline__ int first_job(const Params& p, int begin) {
  const int r = begin % p.ncu;
  return begin + (((int)blockIdx.x - r) % p.ncu + p.ncu) % p.ncu;
}

// Up/gate jobs: the shared expert's tiles come first, then rt_tiles tiles
// per routed group; a down job names its group.  The group and tile are
// derived once on entering a phase and then advanced incrementally.
__device__ inline void settle(const Params& p, const Sched& s, It& c) {
  for (;;) {
    if (c.phase == 0) {
      c.g = 0;
      c.tile = c.j;
      if (c.j < s.sh_tiles) return;
      c.phase = 1;
      c.j = first_job(p, s.sh_tiles);
      c.g = p.n_shared + (c.j - s.sh_tiles) / s.rt_tiles;
      c.tile = (c.j - s.sh_tiles) % s.rt_tiles;
      continue;
    }
    if (c.phase == 1) {
      if (c.j < s.n_jobs) return;
      c.phase = 2;
      c.j = 0;
      c.rt = s.narrow ? wave_id() % s.nrt_p : 0;
      c.tile = 0;
      continue;
    }
    c.g = c.j;
    if (c.phase == 2 && (c.rt >= s.nrt || c.j >= s.G)) c.phase = 3;
    return;
  }
}

__device__ inline void next_job(const Params& p, const Sched& s, It& c) {
  if (c.phase == 0) {
    c.j += p.ncu;
  } else if (c.phase == 1) {
    c.j += p.ncu;
    c.tile += p.ncu;
    while (c.tile >= s.rt_tiles) {
      c.tile -= s.rt_tiles;
      ++c.g;
    }
  } else if (s.narrow) {
    ++c.j;
  } else if (++c.rt >= s.nrt) {
    c.rt = 0;
    ++c.j;
  }
  settle(p, s, c);
}

__device__ __forceinline__ bool shared_group(const Params& p, int g) { return p.n_shared && g == 0; }
__device__ __forceinline__ int job_kdim(const Params& p, const It& c) {
  // (fields taken through uni(): see arg_ptr)
  const int H = uni(p.H), I = uni(p.I), Is = uni(p.Is);
  return c.phase <= 1 ? H : (shared_group(p, c.g) ? Is : I);
}
// This wave's K-blocks of a job: k0 + step*i, i < n.  Up/gate jobs split
// their K-blocks over all 8 waves (k0 = w, step 8).  A down tile belongs to
// the wpt waves w with w % nrt_p == tile, which split its K-blocks
// (k0 = w / nrt_p, step wpt); the other waves have no items in it.
struct KRange {
  int k0, step, n;
};
__device__ __forceinline__ KRange job_krange(const Params& p, const Sched& s, const It& c) {
  const int w = wave_id(), nkb = job_kdim(p, c) >> 7;
  KRange r;
  if (c.phase <= 1) {
    r.k0 = w;
    r.step = kWaves;
  } else {
    r.k0 = w % s.nrt_p == c.rt ? w / s.nrt_p : nkb;
    r.step = s.wpt;
  }
  r.n = uni(nkb > r.k0 ? (nkb - 1 - r.k0) / r.step + 1 : 0);
  r.k0 = uni(r.k0);
  r.step = uni(r.step);
  return r;
}
__device__ __forceinline__ int job_nlive(const Sched& s, const It& c) {
  return c.phase == 2 ? (s.hc - 16 * c.rt < 16 ? s.hc - 16 * c.rt : 16) : 16;
}
// Column c of group g as row*16 + slot.
__device__ __forceinline__ int col_code(const Params& p, const Lds& L, int g, int c) {
  if (shared_group(p, g)) return c * 16 + p.K;
  return (int)lds_ld32(L.cols + lds_ldi_uniform(L.gstart + g) + c);
}

// Column facts of a job's group: its column count and expert (LDS, one
// round trip for a routed group), and this lane's column code in tiles
// 0..NT-1 (a lane past the group's columns takes the last column: MFMA
// columns are independent and that output is never stored).
template <int NT>
__device__ inline void group_cols(const Params& p, const Lds& L, int g, int& ncols, int& eid, int (&code)[NT]) {
  const int lane = threadIdx.x & 63;
  int gstart = 0;
  const bool sh = shared_group(p, g);
  if (sh) {
    ncols = p.T;
    eid = 0;
  } else {
    uint32_t a, b, c;
    asm volatile("ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b), "=&v"(c)
                 : "v"(lds_off(L.gcnt + g)), "v"(lds_off(L.gstart + g)), "v"(lds_off(L.gexp + g))
                 : "memory");
    ncols = uni((int)a);
    gstart = uni((int)b);
    eid = uni((int)c);
  }
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int cc = ct * 16 + (lane & 15) < ncols ? ct * 16 + (lane & 15) : ncols - 1;
    code[ct] = sh ? cc * 16 + p.K : (int)lds_ld32(L.cols + gstart + cc);
  }
}

// Activation offset (elements) of column code `code` for lane group lg:
// x rows for up/gate, mid lines for down.
__device__ __forceinline__ uint32_t act_offset(const Params& p, int kind, int code, int lg) {
  const uint32_t t = kind == 1 ? lmul((uint32_t)(code >> 4), (uint32_t)p.H)
                               : lmul(lmul((uint32_t)(code >> 4), (uint32_t)(p.K + 1)) + (uint32_t)(code & 15),
                                      (uint32_t)p.mid_ld);
  return t + 32u * (uint32_t)lg;
}

// One item in registers.
template <int NPRE>
struct Item {
  u32x4 w0, w1;       // this lane's weights (row lane & 15): FP8 32 bytes, MXFP4 16 (w1 repeats w0)
  u32x4 B[4 * NPRE];  // activations of column tiles 0..NPRE-1 (column lane & 15 of the tile)
  uint32_t s;         // FP8: the K-block's scale of the tile's first (lanes 0-31) or second
                      // (32-63) 128-row block; MXFP4: the lane's row's four E8M0 scales
};

// The fetch side: where this wave's next items come from.
template <int NPRE>
struct Fetch {
  It it;
  int i, n;           // next item of the job, this wave's items in it
  int fmt, live;      // live = 0 past the end of the phase (dummy items)
  int k0, step;       // K-blocks of the job's items: k0 + step*i
  int g, eid;         // group of the last job set up, and its expert
  const uint8_t* wrow;  // this lane's weight row at K offset 0
  const uint8_t* srow;  // this lane's scale row (see Item::s)
  const uint16_t* abase;
  uint32_t act[NPRE];   // this lane's column per prefetched tile: activation offset
};

// Weight and scale rows of a job for this lane.  Up/gate: rows 0..7 are gate
// rows 8t.., 8..15 up rows I+8t..; down: output rows h0+16rt.. (a row past
// the live rows repeats the last live one).
template <int NPRE>
__device__ inline void fetch_job(const Params& p, const Lds& L, const Sched& s, Fetch<NPRE>& f) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const It& c = f.it;
  const bool down = c.phase == 2, sh = shared_group(p, c.g);
  const int iexp = sh ? uni(p.Is) : uni(p.I), kdim = job_kdim(p, c), nlive = job_nlive(s, c);
  const int hb = s.h0 + 16 * c.rt;
  // consecutive jobs of one group (the down tiles of this CU's slice) share
  // the column lookups
  if (c.g != f.g) {
    int ncols, code[NPRE];
    group_cols<NPRE>(p, L, c.g, ncols, f.eid, code);
    f.g = c.g;
    f.abase = down ? arg_ptr(p.mid) : arg_ptr(p.x);
#pragma unroll
    for (int ct = 0; ct < NPRE; ++ct) f.act[ct] = act_offset(p, down ? 2 : 1, code[ct], lg);
  }
  const int eid = f.eid;
  f.fmt = sh ? 0 : uni(p.routed_fmt);
  const KRange kr = job_krange(p, s, c);
  f.n = kr.n;
  f.k0 = kr.k0;
  f.step = kr.step;
  f.i = 0;
  const int wr = down ? hb + (row < nlive ? row : nlive - 1) : (row < 8 ? 8 * c.tile + row : iexp + 8 * c.tile + row - 8);
  const size_t H = p.H, I = p.I, e = (size_t)eid;
  const uint8_t* w;
  const uint8_t* sc;
  if (f.fmt == 0) {
    // FP8 weights [rows][kdim] bytes; fp32 scales [rows/128][kdim/128]
    const float* S;
    if (sh) {
      w = down ? arg_ptr(p.sh_wd) : arg_ptr(p.sh_wgu);
      S = down ? arg_ptr(p.sh_sd) : arg_ptr(p.sh_sgu);
    } else {
      w = down ? arg_ptr(p.wd) + e * H * I : arg_ptr(p.wgu) + e * 2 * I * H;
      S = down ? (const float*)arg_ptr(p.sd) + e * (H / 128) * (I / 128)
               : (const float*)arg_ptr(p.sgu) + e * (2 * I / 128) * (H / 128);
    }
    const int nkb = kdim / 128;
    const int nb_lo = down ? hb / 128 : (8 * c.tile) / 128;
    const int nb_hi = down ? (hb + nlive - 1) / 128 : (iexp + 8 * c.tile) / 128;
    f.wrow = w + (size_t)wr * kdim;
    sc = (const uint8_t*)(S + (size_t)(lane < 32 ? nb_lo : nb_hi) * nkb);
  } else {
    // MXFP4 weights [rows][kdim/2] bytes; E8M0 scales [rows][kdim/32]
    w = down ? arg_ptr(p.wd) + e * H * (I / 2) : arg_ptr(p.wgu) + e * 2 * I * (H / 2);
    const uint8_t* S = down ? (const uint8_t*)arg_ptr(p.sd) + e * H * (I / 32)
                            : (const uint8_t*)arg_ptr(p.sgu) + e * 2 * I * (H / 32);
    f.wrow = w + (size_t)wr * (kdim / 2);
    sc = S + (size_t)wr * (kdim / 32);
  }
  f.srow = sc;
}

// Issues the loads of the fetch side's next item into `it`: always
// 3 + 4*NPRE loads; a dead item (past the phase) loads from x instead.
template <int NPRE>
__device__ __forceinline__ void fetch_item(const Params& p, const Fetch<NPRE>& f, Item<NPRE>& it) {
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  const int kb = f.live ? f.k0 + f.step * f.i : 0;
  const int kbytes = f.fmt ? 64 : 128, lbytes = f.fmt ? 16 : 32;
  const uint8_t* wp = f.live ? f.wrow + kb * kbytes + lg * lbytes : (const uint8_t*)p.x;
  const uint8_t* sp = f.live ? f.srow + 4 * kb : (const uint8_t*)p.x;
  const uint16_t* ab = f.live ? f.abase : arg_ptr(p.x);
  it.w0 = ld16(wp);
  it.w1 = ld16(wp + (f.fmt ? 0 : 16));
  it.s = ldg<uint32_t>(sp);
#pragma unroll
  for (int ct = 0; ct < NPRE; ++ct) {
    const uint16_t* a = ab + (f.live ? f.act[ct] + kb * 128 : 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) it.B[4 * ct + m] = ld16(a + 8 * m);
  }
}

// Moves the fetch side one item on, over jobs this wave has no items in,
// and stops (dead items) at phase `stop`.
template <int NPRE>
__device__ inline void fetch_next(const Params& p, const Lds& L, const Sched& s, Fetch<NPRE>& f, int stop) {
  f.live = uni(f.live);
  if (!f.live) return;
  f.i = uni(f.i) + 1;
  f.n = uni(f.n);
  while (f.i >= f.n) {
    next_job(p, s, f.it);
    uni(f.it);
    if (f.it.phase >= stop) {
      f.live = 0;
      return;
    }
    fetch_job(p, L, s, f);
  }
}

template <int NPRE>
__device__ inline void fetch_start(const Params& p, const Lds& L, const Sched& s, Fetch<NPRE>& f, It start, int stop) {
  f.it = start;
  f.live = start.phase < stop;
  f.fmt = 0;
  f.g = -1;
  f.eid = 0;
  if (!f.live) return;
  fetch_job(p, L, s, f);
  while (f.n == 0) {
    next_job(p, s, f.it);
    if (f.it.phase >= stop) {
      f.live = 0;
      return;
    }
    fetch_job(p, L, s, f);
  }
}

// The multiplying side's view of its current job.
template <int NPRE>
struct Eat {
  It it;
  int i, n;
  int kind;     // 1 up/gate, 2 down
  int g;        // group of the job
  int fmt, tile, rt, ncols, nct, nlive;
  int split;    // FP8: MFMA output rows (4*lg + q) below it take the first block scale
  int k0, step; // K-blocks of the items
  const uint16_t* abase;
  uint32_t act[max_tiles<NPRE>()];  // this lane's column per tile (tiles >= NPRE are loaded when used)
};

template <int NPRE>
__device__ inline void eat_job(const Params& p, const Lds& L, const Sched& s, Eat<NPRE>& e) {
  const int lg = (threadIdx.x & 63) >> 4;
  const It& c = e.it;
  e.kind = c.phase <= 1 ? 1 : 2;
  e.fmt = shared_group(p, c.g) ? 0 : uni(p.routed_fmt);
  e.tile = c.phase <= 1 ? c.tile : 0;
  e.rt = c.phase == 2 ? c.rt : 0;
  e.nlive = job_nlive(s, c);
  const KRange kr = job_krange(p, s, c);
  e.n = kr.n;
  e.k0 = kr.k0;
  e.step = kr.step;
  e.i = 0;
  if (e.kind == 1) {
    e.split = 8;  // rows 0..7 of the MFMA tile are gate rows, 8..15 up rows
  } else {
    // a 16-row down tile spans at most two 128-row scale blocks
    const int hb = s.h0 + 16 * e.rt;
    e.split = (hb / 128 + 1) * 128 - hb;
  }
  // consecutive jobs of one group (the down tiles of this CU's slice, within
  // one phase) have the same columns
  if (c.g == e.g) return;
  e.g = c.g;
  int eid, code[max_tiles<NPRE>()];
  group_cols<max_tiles<NPRE>()>(p, L, c.g, e.ncols, eid, code);
  e.nct = (e.ncols + 15) >> 4;
  e.abase = e.kind == 1 ? arg_ptr(p.x) : arg_ptr(p.mid);
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) e.act[ct] = act_offset(p, e.kind, code[ct], lg);
}

// Multiplies one item into acc[ct].  FP8: a 4-MFMA block sum, then times the
// 128x128 block scale of the output row; MXFP4: the E8M0 scale is folded
// into the exact bf16 conversion.
template <int F, int NPRE>
__device__ inline void eat_item(const Eat<NPRE>& e, const Item<NPRE>& it, f32x4* acc) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int kb = e.k0 + e.step * e.i;
  bf16x8 A[4];
  float s_lo = 1.f, s_hi = 1.f;
  if (F == 0) {
    A[0] = e4m3x8_to_bf16(it.w0[0], it.w0[1]);
    A[1] = e4m3x8_to_bf16(it.w0[2], it.w0[3]);
    A[2] = e4m3x8_to_bf16(it.w1[0], it.w1[1]);
    A[3] = e4m3x8_to_bf16(it.w1[2], it.w1[3]);
    s_lo = __int_as_float(__builtin_amdgcn_readlane((int)it.s, 0));
    s_hi = __int_as_float(__builtin_amdgcn_readlane((int)it.s, 32));
  } else {
    const float sc = e8m0_to_f32((it.s >> (8 * lg)) & 0xffu);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w0[m], sc);
  }
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
    if (ct < e.nct) {
      u32x4 Bl[4];
      const u32x4* B = it.B + 4 * (ct < NPRE ? ct : 0);
      if (ct >= NPRE) {
        const uint16_t* a = e.abase + e.act[ct] + kb * 128;
#pragma unroll
        for (int m = 0; m < 4; ++m) Bl[m] = ld16(a + 8 * m);
        B = Bl;
      }
      if (F == 0) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) t = mfma16(A[m], __builtin_bit_cast(bf16x8, B[m]), t);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ct][q] = fmaf(t[q], 4 * lg + q < e.split ? s_lo : s_hi, acc[ct][q]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[ct] = mfma16(A[m], __builtin_bit_cast(bf16x8, B[m]), acc[ct]);
      }
    }
  }
}

// mid = silu(gate) * up in fp32 (one expression for both layouts).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Job-end reductions.  At the end of a job every wave stores its partial
// tiles into partial slot (job % slots) and raises its part count; it never
// waits for the others there.  Job j is summed by its owner wave (j mod 8)
// later: at the owner's next job end, at the up/gate -> down hand-over, or
// while the owner waits for a slot.  The sum runs over the waves in order
// 0..7, exactly as a workgroup-wide reduction would.  A slot is reused for
// job j only after job j - slots was summed out of it.
struct Owned {
  int jc;       // the job's index in this CU's sequence, -1 when none
  int kind, g, tile, rt, ncols, nct, nlive;
};

// Eight waves' partial f32x4 of one lane, 1 KB apart, in one round trip.
__device__ __forceinline__ void lds_ld_wave_partials(const float* t, u32x4 (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(lds_off(t))
      : "memory");
}

__device__ __forceinline__ const float* red_slot(const Lds& L, int T, int jc) {
  return L.red + (size_t)(jc % red_slots(T)) * red_tiles(T) * (kRedTileBytes / 4);
}

// Sums the owned job out of its slot.  Lane l holds MFMA rows 4*(l>>4)+q of
// column (l & 15) in every wave's partial.  Up/gate: rows 0..7 are gate
// rows, 8..15 (32 lanes on) the matching up rows; lanes 0..31 each finish
// four intermediates, mid = silu(gate) * up rounded to bf16.  Down: every
// lane finishes its four rows into the LDS products.
template <int NPRE>
__device__ inline void sum_job(const Params& p, const Lds& L, const Owned& o) {
  const int lane = threadIdx.x & 63;
  const float* base = red_slot(L, p.T, o.jc);
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
    if (ct < o.nct) {
      const float* t = base + (size_t)ct * (kRedTileBytes / 4);
      const int col = ct * 16 + (lane & 15);
      const int code = col_code(p, L, o.g, col < o.ncols ? col : o.ncols - 1);
      if (o.kind == 1) {
        if (lane < 32) {
          u32x4 v[8];
          float gs[4], us[4];
          lds_ld_wave_partials(t + (size_t)lane * 4, v);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gs[q] = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) gs[q] += __uint_as_float(v[w][q]);
          }
          lds_ld_wave_partials(t + (size_t)(lane + 32) * 4, v);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            us[q] = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) us[q] += __uint_as_float(v[w][q]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = gs[q], u = us[q];
            if (col < o.ncols) {
              const float m = swiglu(g, u);
              if (!isfinite(m)) set_err(p.err, kErrMid);
              const int i = 4 * (lane >> 4) + q;
              p.mid[((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.mid_ld + 8 * o.tile + i] =
                  (uint16_t)f32_to_bf16_rne(m);
            }
          }
        }
      } else {
        u32x4 pv[8];
        lds_ld_wave_partials(t + (size_t)lane * 4, pv);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) v += __uint_as_float(pv[w][q]);
          const int i = 4 * (lane >> 4) + q;
          if (i < o.nlive && col < o.ncols) {
            if (!isfinite(v)) set_err(p.err, kErrMid);
            lds_st32(L.pbuf + ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.hs + 16 * o.rt + i,
                     __float_as_uint(v));
          }
        }
      }
    }
  }
}

// Sums the owned job when every wave's partials are in (or waits for them
// when `block`), then releases its slot.
template <int NPRE>
__device__ inline void service(const Params& p, const Lds& L, Owned& o, bool block, bool& ok) {
  o.jc = uni(o.jc);
  if (o.jc < 0) return;
  if (block) lds_wait<8>(p, L.ctl + kCtlPart, (uint32_t)(o.jc + 1), ok);
  else if (ok && (int)lds_min<8>(L.ctl + kCtlPart) < o.jc + 1) return;
  sum_job<NPRE>(p, L, o);
  lds_st32(L.ctl + kCtlSlot + o.jc % red_slots(p.T), (uint32_t)(o.jc + 1));
  o.jc = -1;
}

// End of job jc for this wave: wait for its slot (summing an owned job
// meanwhile), store the partial tiles, raise the part count, sum an older
// owned job if its partials are all in, and take ownership of jc when it is
// this wave's.
template <int NPRE>
__device__ inline void job_end(const Params& p, const Lds& L, const Eat<NPRE>& e, f32x4* acc, int jc, Owned& own,
                               bool& ok) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int ns = red_slots(p.T);
  if (jc >= ns) {
    const uint32_t target = (uint32_t)(jc - ns + 1);
    const uint32_t* sd = L.ctl + kCtlSlot + jc % ns;
    int spins = 0;
    while (ok && lds_min<1>(sd) < target) {
      service<NPRE>(p, L, own, false, ok);
      if (++spins > kSpinLimit) {
        set_err(p.err, kErrTimeout);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  float* base = (float*)red_slot(L, p.T, jc);
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct)
    if (ct < e.nct)
      lds_st128(base + (size_t)ct * (kRedTileBytes / 4) + ((size_t)wave * 64 + lane) * 4,
                __builtin_bit_cast(u32x4, acc[ct]));
  lds_st32(L.ctl + kCtlPart + wave, (uint32_t)(jc + 1));
  service<NPRE>(p, L, own, false, ok);
  if (jc % kWaves == wave) {
    service<NPRE>(p, L, own, true, ok);  // the previous owned job, 8 jobs back
    own.jc = jc;
    own.kind = e.kind;
    own.g = e.it.g;
    own.tile = e.tile;
    own.rt = e.rt;
    own.ncols = e.ncols;
    own.nct = e.nct;
    own.nlive = e.nlive;
  }
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// The two waves of a SIMD (w and w ^ 4) have the same work, but the issue
// arbiter favours the older one, which would then finish its phase early and
// leave the newer one streaming alone.  At every job end the wave that is
// ahead of its partner lowers its priority.
__device__ __forceinline__ void balance(const Lds& L, int jc) {
  const int wave = wave_id();
  lds_st32(L.ctl + kCtlProg + wave, (uint32_t)jc);
  const int other = (int)lds_min<1>(L.ctl + kCtlProg + (wave ^ 4));
  if (jc > other) __builtin_amdgcn_s_setprio(0);
  else __builtin_amdgcn_s_setprio(2);
}

// Moves the multiplying side on after an item; at the end of a job (and for
// every following job this wave has no items in) runs the job end.  Returns
// false once the phase is done.
template <int NPRE>
__device__ inline bool eat_next(const Params& p, const Lds& L, const Sched& s, Eat<NPRE>& e, f32x4* acc, int& jc,
                                Owned& own, bool& ok, int stop) {
  e.i = uni(e.i) + 1;
  e.n = uni(e.n);
  while (e.i >= e.n) {
    job_end<NPRE>(p, L, e, acc, jc++, own, ok);
    MOE_JSTAMP(p, jc - 1);
    balance(L, jc);
    next_job(p, s, e.it);
    uni(e.it);
    if (e.it.phase >= stop) return false;
    eat_job(p, L, s, e);
  }
  return true;
}

// One phase (up/gate, or down) of the stream: a D-deep register pipeline.
// Each step multiplies item n out of ring slot n % D and refills that slot
// with item n + D.
template <int NPRE, int FMT>
__device__ __forceinline__ void run_phase(const Params& p, const Lds& L, const Sched& s, It start, int stop, f32x4* acc,
                                 int& jc, Owned& own, bool& ok) {
  constexpr int D = depth<NPRE>();
  if (start.phase >= stop) return;
  Fetch<NPRE> f;
  fetch_start(p, L, s, f, start, stop);
  Item<NPRE> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    fetch_item(p, f, ring[d]);
    fetch_next(p, L, s, f, stop);
  }
  Eat<NPRE> e;
  e.it = start;
  e.g = -1;
  eat_job(p, L, s, e);
  // jobs this wave has no items in still end (with zero partials)
  bool more = true;
  while (e.n == 0 && more) {
    job_end<NPRE>(p, L, e, acc, jc++, own, ok);
    next_job(p, s, e.it);
    if (e.it.phase >= stop) more = false;
    else eat_job(p, L, s, e);
  }
  // The loop is left only after a whole round of D slots (the rest of the
  // round refills with dead loads), so every path to an item's wait has
  // issued the same D-1 items since; an exit in mid-round would make the
  // compiler's wait counting assume fewer and drain the ring.
  bool done = !more;
  if (!done) {
    for (;;) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (!done) {
          if (e.fmt == 0) eat_item<0>(e, ring[d], acc);
          else eat_item<FMT>(e, ring[d], acc);
        }
        fetch_item(p, f, ring[d]);
        fetch_next(p, L, s, f, stop);
        if (!done) done = !eat_next(p, L, s, e, acc, jc, own, ok, stop);
      }
      if (done) break;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the dead items' loads
  __builtin_amdgcn_s_setprio(0);
}

// ------------------------------------------------------------------ narrow stream
//
// Batches of at most 16 rows (one 16-column MFMA tile per group).  A wave's
// items run through a D-deep register ring: each step multiplies the oldest
// item, refills its slot with the item D later and counts; only a job
// change on either side does more.  At a job end the wave stores its
// partial tile into its own part of LDS and never waits for another wave.

// A job as the narrow stream sees it, built once per call for every job of
// this CU (see build_jobs).  Lanes add their row, K-block and column.
struct JobDesc {
  uint64_t wb;        // weights of the job's row 0 (up/gate: gate row 8t; down: the expert's W_down)
  uint64_t sb;        // block scales of that row (FP8 up/gate: its 128-row block row; MXFP4: its row)
  uint32_t tile;      // up/gate: the 8-intermediate tile
  uint32_t jump;      // up/gate: rows between lane row 7 (gate) and lane row 8 (up), minus one
  uint32_t shi;       // FP8 up/gate: scale bytes from the gate rows' block row to the up rows'; MXFP4: scale bytes per row
  int32_t nkb;        // K-blocks
  int32_t fmt;        // 0 FP8, 1 MXFP4
  int32_t ncols;      // the group's columns
  int32_t cbase;      // its first column in the column table
  int32_t spare;
};
static_assert(sizeof(JobDesc) == 48, "three 16-byte LDS reads");

__device__ inline JobDesc read_desc(const Lds& L, int k) {
  u32x4 a, b, c;
  asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:16\n\tds_read_b128 %2, %3 offset:32\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b), "=&v"(c)
               : "v"(lds_off(L.jd + k))
               : "memory");
  JobDesc d;
  d.wb = ((uint64_t)(uint32_t)uni((int)a[1]) << 32) | (uint32_t)uni((int)a[0]);
  d.sb = ((uint64_t)(uint32_t)uni((int)a[3]) << 32) | (uint32_t)uni((int)a[2]);
  d.tile = (uint32_t)uni((int)b[0]);
  d.jump = (uint32_t)uni((int)b[1]);
  d.shi = (uint32_t)uni((int)b[2]);
  d.nkb = uni((int)b[3]);
  d.fmt = uni((int)c[0]);
  d.ncols = uni((int)c[1]);
  d.cbase = uni((int)c[2]);
  d.spare = 0;
  return d;
}

// The descriptor of an up/gate job (tile `tile` of the expert's 8-row gate
// and up tiles) or of a down job (the expert's whole W_down).
__device__ inline JobDesc make_desc(const Params& p, bool up, bool sh, int e, int tile, int ncols, int cbase) {
  const size_t H = p.H, I = p.I;
  JobDesc d;
  const int iexp = sh ? p.Is : p.I;
  const int kdim = up ? p.H : iexp;
  d.fmt = sh ? 0 : p.routed_fmt;
  d.nkb = kdim / 128;
  d.ncols = ncols;
  d.cbase = cbase;
  d.spare = 0;
  d.jump = up ? iexp - 8 : 0;
  d.tile = (uint32_t)tile;
  const uint8_t* w;
  const uint8_t* S;
  if (d.fmt == 0) {
    if (sh) {
      w = up ? p.sh_wgu : p.sh_wd;
      S = (const uint8_t*)(up ? p.sh_sgu : p.sh_sd);
    } else {
      w = up ? p.wgu + (size_t)e * 2 * I * H : p.wd + (size_t)e * H * I;
      S = up ? (const uint8_t*)p.sgu + 4 * (size_t)e * (2 * I / 128) * (H / 128)
             : (const uint8_t*)p.sd + 4 * (size_t)e * (H / 128) * (I / 128);
    }
    if (up) {
      const int nb_lo = (8 * tile) / 128, nb_hi = (iexp + 8 * tile) / 128;
      w += (size_t)8 * tile * kdim;
      S += 4 * (size_t)nb_lo * d.nkb;
      d.shi = 4u * (uint32_t)((nb_hi - nb_lo) * d.nkb);
    } else {
      d.shi = 0;
    }
  } else {
    d.shi = kdim / 32;
    w = up ? p.wgu + (size_t)e * 2 * I * (H / 2) : p.wd + (size_t)e * H * (I / 2);
    S = up ? (const uint8_t*)p.sgu + (size_t)e * 2 * I * (H / 32) : (const uint8_t*)p.sd + (size_t)e * H * (I / 32);
    if (up) {
      w += (size_t)8 * tile * (kdim / 2);
      S += (size_t)8 * tile * d.shi;
    }
  }
  d.wb = (uint64_t)w;
  d.sb = (uint64_t)S;
  return d;
}

// Up/gate job j of the step: the shared tiles, then rt_tiles tiles per
// routed group.  Sets its group and tile.
__device__ __forceinline__ void up_job(const Params& p, const Sched& s, int j, int& g, int& tile) {
  if (j < s.sh_tiles) {
    g = 0;
    tile = j;
  } else {
    g = p.n_shared + (j - s.sh_tiles) / s.rt_tiles;
    tile = (j - s.sh_tiles) % s.rt_tiles;
  }
}

// Up/gate jobs of a narrow call: CU c takes jobs c + q*ncu (local job q),
// as in the wide stream.  Inside the CU a job is cut into chunks, one per
// K-phase w (K-blocks w + 8i, the blocks wave w takes in the wide stream),
// and the waves claim chunks in order from an LDS counter.  A chunk's
// partial is the same sum whichever wave forms it, so the job's sum over its
// K-phases in order does not depend on which wave did what, and waves that
// stream faster take more chunks.


// The narrow stream's state and the tables of this CU's shared-expert jobs
// (local jobs 0..nS-1; they need no routing).  Whole workgroup, plain
// per-thread LDS accesses; the caller synchronises.
// This CU's shared-expert up/gate jobs (dealt c, c + ncu, ...).
__device__ __forceinline__ int shared_jobs_here(const Params& p) {
  const int sh_tiles = p.n_shared ? p.Is / 8 : 0;
  return (int)blockIdx.x < sh_tiles ? (sh_tiles - 1 - (int)blockIdx.x) / p.ncu + 1 : 0;
}

__device__ inline void stream_init(const Params& p, const Lds& L, int nS) {
  const int tid = threadIdx.x;
  for (int k = tid; k < nS; k += kThreads)
    L.jd[k] = make_desc(p, true, true, 0, (int)blockIdx.x + k * p.ncu, p.T, 0);
  if (p.n_shared && tid < p.T) {
    L.cols[tid] = tid * 16 + p.K;
    L.cgrp[tid] = 0;
  }
  if (tid < kPuWin) {
    L.wcnt[tid] = 0u;
    L.wgen[tid] = 0u;
  }
  if (tid == 0) {
    *L.ccnt = 0u;
    L.misc[kMiscReady] = 0;
    L.misc[kMiscRouted] = 0;
    L.misc[kMiscPolled] = 0;
  }
}

// The tables that need the routing: the routed up/gate jobs (local jobs
// nS..nU-1) and one down job per group at qcap + g, written by threads
// first, first + stride, ...; then nU.
// PART: 1 the up/gate jobs and nU, 2 the down jobs, 3 both.
template <int PART = 3>
__device__ inline void routed_tables(const Params& p, const Lds& L, const Sched& s, int nS, int nU, int first,
                                     int stride) {
  if (PART & 1) {
    for (int k = nS + first; k < nU; k += stride) {
      int g, tile;
      up_job(p, s, (int)blockIdx.x + k * p.ncu, g, tile);
      const bool sh = shared_group(p, g);
      L.jd[k] = make_desc(p, true, sh, sh ? 0 : L.gexp[g], tile, sh ? p.T : L.gcnt[g], sh ? 0 : L.gstart[g]);
    }
  }
  if (PART & 2) {
    for (int g = first; g < s.G; g += stride) {
      const bool sh = shared_group(p, g);
      L.jd[p.qcap + g] = make_desc(p, false, sh, sh ? 0 : L.gexp[g], 0, sh ? p.T : L.gcnt[g], sh ? 0 : L.gstart[g]);
    }
  }
  if ((PART & 1) && first == 0) L.misc[kMiscNU] = nU;
}

// Per-wave constants of a phase (KIND 1 up/gate, 2 down).  Up/gate: every
// wave takes K-blocks w + 8i of each job, rows 0..7 of a tile are gate rows
// and 8..15 up rows.  Down: wave w takes tile rt = w % nrt_p of the CU's
// slice, rows hb.. (nlive live), and K-blocks w / nrt_p + wpt*i.
struct PhaseN {
  int k0, lstep;  // this wave's K-blocks: k0 + (i << lstep)
  int hb, nlive;  // down: first row of this wave's tile and its live rows
  int split;      // FP8: MFMA output rows (4*lg + q) below it take the first scale block row
  int dnb;        // FP8 down: block rows between the tile's first and last live row (0 or 1)
  int rt;         // down: this wave's tile
  int nw;         // up/gate: waves with items (min(K-blocks, 8))
};
template <int KIND>
__device__ __forceinline__ int ph_k0(const PhaseN& ph) { return KIND == 1 ? wave_id() : ph.k0; }
template <int KIND>
__device__ __forceinline__ int ph_lstep(const PhaseN& ph) { return KIND == 1 ? 3 : ph.lstep; }
template <int KIND>
__device__ __forceinline__ int ph_split(const PhaseN& ph) { return KIND == 1 ? 8 : ph.split; }

template <int KIND>
__device__ __forceinline__ int job_items(const PhaseN& ph, int nkb) {
  const int k0 = ph_k0<KIND>(ph);
  return nkb > k0 ? ((nkb - 1 - k0) >> ph_lstep<KIND>(ph)) + 1 : 0;
}

// The fetch side: byte offsets of this lane's next item from uniform bases.
struct FetchN {
  int k;                         // next job to set up (down)
  int nch;                       // up/gate: chunks claimed by this wave
  int nu;                        // up/gate: the CU's job count once the routed tables are in (else -1)
  int cnt;                       // items fetched so far
  int left;                      // items left in the job (large once past the phase)
  int nstep;                     // K-blocks per item step (0 once past the phase)
  int fmt;                       // 0 FP8, 1 MXFP4
  const uint8_t* wb;             // weights
  const uint8_t* sb;             // block scales
  const uint8_t* ab;             // activations: x or mid
  uint32_t wo, so, ao;           // this lane's offsets of the next item
};

struct ItemN {
  u32x4 w0, w1, B[4];
  uint32_t s;
};

// Column code (row*16 + slot) of this lane's column in a job (a lane past
// the group's columns takes its last one: MFMA columns are independent and
// that output is never stored).
// Activation loads per item, AL = 1, 2 or 4: a job of at most 4*AL columns
// places group column c at MFMA columns G*c..G*c+G-1 (G = 4/AL lanes per
// column), and lane G*c+j loads the 16-B pieces j, j+G, .. of its K-block
// (see act_operand).
template <int AL>
__device__ __forceinline__ int lane_col(int lane) {
  return (lane & 15) >> (AL == 1 ? 2 : AL == 2 ? 1 : 0);
}
template <int AL>
__device__ __forceinline__ int lane_code(const Lds& L, const JobDesc& d) {
  const int col = lane_col<AL>(threadIdx.x);
  return (int)lds_ld32(L.cols + d.cbase + (col < d.ncols ? col : d.ncols - 1));
}

// Sets the fetch side to job descriptor d, whose first item is this wave's
// K-block k0; `code` is this lane's column (row*16 + slot), n its items.
template <int FMT, int KIND, int AL>
__device__ __forceinline__ void fetch_from_desc(const Params& p, const PhaseN& ph, FetchN& f, const JobDesc& d, int k0,
                                                int n, int code) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const int fmt = FMT == 0 ? 0 : d.fmt;
  const uint32_t kb = fmt ? 64u : 128u, lb = fmt ? 16u : 32u;
  const uint32_t lrow = KIND == 1 ? (row < 8 ? row : row + d.jump) : ph.hb + (row < ph.nlive ? row : ph.nlive - 1);
  f.wb = (const uint8_t*)d.wb;
  f.wo = lmul(lrow, (uint32_t)(d.nkb * (fmt ? 64 : 128))) + (uint32_t)k0 * kb + (uint32_t)lg * lb;
  if (fmt == 0) {
    if (KIND == 1) {
      f.sb = (const uint8_t*)d.sb;
      f.so = (lane < 32 ? 0u : d.shi) + 4u * (uint32_t)k0;
    } else {
      f.sb = (const uint8_t*)d.sb + 4 * (size_t)(ph.hb >> 7) * d.nkb;
      f.so = (lane < 32 ? 0u : 4u * (uint32_t)(ph.dnb * d.nkb)) + 4u * (uint32_t)k0;
    }
  } else {
    f.sb = (const uint8_t*)d.sb;
    f.so = lmul(lrow, d.shi) + 4u * (uint32_t)k0;
  }
  // a lane's first piece: j = lane mod G
  f.ao = 2 * act_offset(p, KIND, code, lg) + 256u * (uint32_t)k0 + 16u * (uint32_t)(lane & (4 / AL - 1));
  f.fmt = fmt;
  f.nstep = 1 << ph_lstep<KIND>(ph);
  f.left = n;
}

// Past the last job: dead items load from the start of x (weights and
// scales) and of the phase's own activations, and are never multiplied (f.ab
// stays: a split fill's items still take their activations from it).
// (The fields are stored in the order fetch_from_desc stores them: the
// compiler merges the two paths' stores pairwise, and pairs of different
// fields would leave the fetch side in scratch memory.)
__device__ __forceinline__ void fetch_dead(const Params& p, FetchN& f) {
  f.wb = (const uint8_t*)arg_ptr(p.x);
  f.wo = 0;
  f.sb = (const uint8_t*)arg_ptr(p.x);
  f.so = 0;
  f.ao = 0;
  f.fmt = 0;
  f.nstep = 0;
  f.left = 1 << 30;
}

// Down: moves the fetch side to the next job of [f.k, kend) with items for
// this wave, or past the end.
template <int FMT, int KIND, int AL>
__device__ inline void fetch_next_n(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int kend) {
  for (; f.k < kend; ++f.k) {
    const JobDesc d = read_desc(L, f.k);
    const int n = job_items<KIND>(ph, d.nkb);
    if (n == 0) continue;
    ++f.k;
    fetch_from_desc<FMT, KIND, AL>(p, ph, f, d, ph_k0<KIND>(ph), n, lane_code<AL>(L, d));
    return;
  }
  fetch_dead(p, f);
}

// LDS reads through address-space pointers, so that the compiler counts
// them on the right counter (see ldg).
template <class T>
__device__ __forceinline__ T lds_get(const void* a) {
  return *(const __attribute__((address_space(3))) T*)a;
}

// Adds 1 to an LDS word from lane 0 and returns the old value to all lanes.
__device__ __forceinline__ uint32_t lds_inc_lane0(uint32_t* a) {
  uint32_t v = 0;
  if ((threadIdx.x & 63) == 0)
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(a)), "v"(1u) : "memory");
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Up/gate: claims this CU's next chunk c (local job c / nw, K-phase
// c mod nw) and moves the fetch side to it, handing c on to the multiplying
// side; past the end once c / nw reaches the CU's job count (the wave then
// claims no more).  Jobs from nS on wait for the routed tables (bounded).
__device__ __forceinline__ int chunk_job(uint32_t c, int nw) { return nw == kWaves ? (int)(c >> 3) : (int)c / nw; }
template <int FMT, int AL>
__device__ inline void fetch_next_up(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int nS, bool& ok) {
  const uint32_t c = lds_inc_lane0(L.ccnt);
  const int q = chunk_job(c, ph.nw), kp = (int)c - q * ph.nw;
  if (q >= nS && f.nu < 0) {
    lds_wait<1>(p, (const uint32_t*)L.misc + kMiscReady, 1u, ok);
    f.nu = ok ? lds_ldi_uniform(L.misc + kMiscNU) : 0;
  }
  if (q < (q < nS ? nS : f.nu)) {
    const JobDesc d = read_desc(L, q);
    lds_st32(L.cfifo + wave_id() * 8 + (f.nch & 7), c);
    f.nch = f.nch + 1;
    fetch_from_desc<FMT, 1, AL>(p, ph, f, d, kp, ((d.nkb - 1 - kp) >> 3) + 1, lane_code<AL>(L, d));
    return;
  }
  fetch_dead(p, f);
}

// kend: up/gate, the CU's shared-expert job count; down, the end of its
// job range.
template <int FMT, int KIND, int AL>
__device__ __forceinline__ void fetch_next_any(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int kend,
                                               bool& ok) {
  if (KIND == 1) fetch_next_up<FMT, AL>(p, L, ph, f, kend, ok);
  else fetch_next_n<FMT, KIND, AL>(p, L, ph, f, kend);
}

template <int FMT>
__device__ __forceinline__ void fetch_weights_n(const FetchN& f, ItemN& it) {
  const uint8_t* w = f.wb + f.wo;
  it.w0 = ldg<u32x4>(w);
  it.w1 = ldg<u32x4>(w + (FMT == 0 || f.fmt == 0 ? 16 : 0));
  it.s = ldg<uint32_t>(f.sb + f.so);
}
// Activations: AL loads of 16 B per lane, pieces j + G*i (the load
// instructions, not the bytes, are what the vector memory path pays for).
template <int AL>
__device__ __forceinline__ void fetch_acts_n(const uint8_t* ab, uint32_t ao, ItemN& it) {
  const uint8_t* a = ab + ao;
#pragma unroll
  for (int i = 0; i < AL; ++i) it.B[i] = ldg<u32x4>(a + 16 * (4 / AL) * i);
}
template <int FMT, int AL>
__device__ __forceinline__ void fetch_item_n(const FetchN& f, ItemN& it) {
  fetch_weights_n<FMT>(f, it);
  fetch_acts_n<AL>(f.ab, f.ao, it);
}

template <int FMT>
__device__ __forceinline__ void fetch_adv_n(FetchN& f) {
  const uint32_t n = (uint32_t)uni(f.nstep);
  f.wo += n * (FMT == 0 || f.fmt == 0 ? 128u : 64u);
  f.so += 4u * n;
  f.ao += 256u * n;
  f.left = uni(f.left) - 1;
  f.cnt = uni(f.cnt) + 1;
}

// The multiplying side.
struct EatN {
  int k;
  int nch;         // up/gate: chunks taken from the fetch side
  int q;           // up/gate: the local job being multiplied
  int left;        // items left in the job
  int fmt;         // 0 FP8, 1 MXFP4
  uint32_t pidx;   // this lane's partial (floats from L.pbuf); only stored when pst
  bool pst;        // this lane's column is one of the group's
};

// Down: moves the multiplying side to its next job of [e.k, kend) with
// items; false at the end.
template <int FMT, int KIND, int AL>
__device__ inline bool eat_next_n(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, int kend) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane_col<AL>(lane);
  for (; e.k < kend; ++e.k) {
    const JobDesc d = read_desc(L, e.k);
    const int n = job_items<KIND>(ph, d.nkb);
    if (n == 0) continue;
    ++e.k;
    e.left = n;
    e.fmt = FMT == 0 ? 0 : d.fmt;
    e.pst = col < d.ncols && (lane & (4 / AL - 1)) == 0;
    const int code = lane_code<AL>(L, d);
    e.pidx = lmul(lmul((uint32_t)ph.k0 * (uint32_t)p.T + (uint32_t)(code >> 4), (uint32_t)(p.K + 1)) +
                      (uint32_t)(code & 15),
                  (uint32_t)p.pitch) +
             16u * (uint32_t)ph.rt + 4u * (uint32_t)lg;
    return true;
  }
  return false;
}

// Up/gate: moves the multiplying side to the next chunk the fetch side has
// set up (fnch: chunks it has claimed); false at the end.  The partial goes
// to window q mod kPuWin, K-phase row kp, the lane's column.
template <int FMT, int AL>
__device__ inline bool eat_next_up(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, int fnch) {
  if (e.nch >= fnch) return false;
  const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane_col<AL>(lane);
  const uint32_t c = (uint32_t)lds_ldi_uniform((const int32_t*)L.cfifo + wave_id() * 8 + (e.nch & 7));
  e.nch = e.nch + 1;
  const int q = chunk_job(c, ph.nw), kp = (int)c - q * ph.nw;
  const JobDesc d = read_desc(L, q);
  e.q = q;
  e.left = ((d.nkb - 1 - kp) >> 3) + 1;
  e.fmt = FMT == 0 ? 0 : d.fmt;
  e.pst = col < d.ncols && (lane & (4 / AL - 1)) == 0;
  e.pidx = ((((uint32_t)q & (kPuWin - 1)) * kWaves + (uint32_t)kp) * (uint32_t)p.T + (uint32_t)col) * 16u +
           4u * (uint32_t)lg;
  return true;
}

// Up/gate job q is complete in partial window win (waves 0..nw-1 stored):
// every (column, intermediate) is summed over the 8 waves in order (a wave
// without items adds zero), gate and up, and its SwiGLU value goes to mid as
// bf16.  One wave; lane = (column, pair of intermediates).
__device__ inline void up_reduce_job(const Params& p, const Lds& L, int q, int win, int nw) {
  const JobDesc d = read_desc(L, q);
  const int lane = threadIdx.x & 63, col = lane >> 2, i2 = 2 * (lane & 3);
  if (col < d.ncols) {
    const size_t wstride = (size_t)p.T * 16;
    const float* pu = L.pbuf + ((size_t)win * kWaves * p.T + col) * 16 + i2;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f32x2 gv = {0.f, 0.f}, uv = {0.f, 0.f};
      if (w < nw) {
        gv = lds_get<f32x2>(pu + w * wstride);
        uv = lds_get<f32x2>(pu + w * wstride + 8);
      }
      g0 += gv[0];
      g1 += gv[1];
      u0 += uv[0];
      u1 += uv[1];
    }
    const float m0 = swiglu(g0, u0), m1 = swiglu(g1, u1);
    if (!isfinite(m0) || !isfinite(m1)) set_err(p.err, kErrMid);
    const int code = lds_get<int32_t>(L.cols + d.cbase + col);
    st_agent<uint32_t>(p.mid + ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.mid_ld + 8 * d.tile + i2,
                       f32_to_bf16_rne(m0) | (f32_to_bf16_rne(m1) << 16));
  }
}

// The end of a chunk of up/gate job e.q: once the window's previous job is
// summed, store the chunk's partial tile and arrive; the wave that ends the
// job's last (nw-th) chunk sums the job and frees the window.
__device__ inline void up_job_end(const Params& p, const Lds& L, const EatN& e, const f32x4& acc, int nw, bool& ok) {
  const int win = e.q & (kPuWin - 1);
  lds_wait<1>(p, L.wgen + win, (uint32_t)(e.q / kPuWin), ok);
  if (e.pst) lds_st128(L.pbuf + e.pidx, __builtin_bit_cast(u32x4, acc));
  if (lds_inc_lane0(L.wcnt + win) == (uint32_t)nw - 1) {
    up_reduce_job(p, L, e.q, win, nw);
    lds_st32(L.wcnt + win, 0u);
    lds_st32(L.wgen + win, (uint32_t)(e.q / kPuWin + 1));
  }
}

// MFMA m's activations: piece m is load m / G of the column's lane m mod G,
// broadcast over the column's G lanes by a DPP quad permutation (G = 4:
// quad_perm(m,m,m,m); G = 2: (0,0,2,2) or (1,1,3,3)).
template <int AL>
__device__ __forceinline__ bf16x8 act_operand(const ItemN& it, int m) {
  if (AL == 4) return __builtin_bit_cast(bf16x8, it.B[m]);
  constexpr int G = 4 / AL;
  u32x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = (int)it.B[m / G][i];
    int r;
    if (G == 4) {
      switch (m) {
        case 0: r = __builtin_amdgcn_update_dpp(0, v, 0x00, 0xF, 0xF, false); break;
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false); break;
      }
    } else if ((m & 1) == 0) {
      r = __builtin_amdgcn_update_dpp(0, v, 0xA0, 0xF, 0xF, false);
    } else {
      r = __builtin_amdgcn_update_dpp(0, v, 0xF5, 0xF, 0xF, false);
    }
    b[i] = (uint32_t)r;
  }
  return __builtin_bit_cast(bf16x8, b);
}

template <int F, int AL>
__device__ __forceinline__ void eat_item_n(int split, int lg, const ItemN& it, f32x4& acc) {
  bf16x8 A[4];
  if (F == 0) {
    A[0] = e4m3x8_to_bf16(it.w0[0], it.w0[1]);
    A[1] = e4m3x8_to_bf16(it.w0[2], it.w0[3]);
    A[2] = e4m3x8_to_bf16(it.w1[0], it.w1[1]);
    A[3] = e4m3x8_to_bf16(it.w1[2], it.w1[3]);
    const float s_lo = __int_as_float(__builtin_amdgcn_readlane((int)it.s, 0));
    const float s_hi = __int_as_float(__builtin_amdgcn_readlane((int)it.s, 32));
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) t = mfma16(A[m], act_operand<AL>(it, m), t);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(t[q], 4 * lg + q < split ? s_lo : s_hi, acc[q]);
  } else {
    const float sc = e8m0_to_f32((it.s >> (8 * lg)) & 0xffu);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w0[m], sc);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = mfma16(A[m], act_operand<AL>(it, m), acc);
  }
}

// One phase of the narrow stream over jobs [k, kend) of the job tables, in
// pieces: ring_open sets the fetch side to the first job, ring_fill issues
// the first D items (all loads, or weights and scales only, the
// activations following in ring_fill_acts), and ring_run multiplies and
// refills until the last job has ended.  Partials go to LDS, which must be
// zero where this wave has no items.
constexpr int kRingD = 5;   // up/gate (and the default)
constexpr int kRingDD = 6;  // down: its second tile has fewer live rows, so items carry fewer bytes
// up/gate ring depth by activation loads per item (2 loads: 7 measured
// best at 8 rows)
template <int AL>
constexpr int ring_up() { return AL == 2 ? 7 : kRingD; }
template <int D = kRingD>
struct RingN {
  FetchN f;
  ItemN r[D];
  uint32_t aop[D];  // activation offsets of the filled items (split fill)
};

template <int FMT, int KIND, int D, int AL>
__device__ __forceinline__ void ring_open(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int k, int kend,
                                          bool& ok) {
  R.f.k = k;
  R.f.nch = 0;
  R.f.nu = -1;
  R.f.cnt = 0;
  R.f.ab = (const uint8_t*)(KIND == 1 ? arg_ptr(p.x) : arg_ptr(p.mid));
  fetch_next_any<FMT, KIND, AL>(p, L, ph, R.f, kend, ok);
}

// WONLY: weights and scales only (the activation offsets are kept).
template <int FMT, int KIND, bool WONLY, int D, int AL>
__device__ __forceinline__ void ring_fill(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int kend,
                                          bool& ok) {
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (WONLY) {
      fetch_weights_n<FMT>(R.f, R.r[d]);
      R.aop[d] = R.f.ao;
    } else {
      fetch_item_n<FMT, AL>(R.f, R.r[d]);
    }
    fetch_adv_n<FMT>(R.f);
    if (R.f.left == 0) fetch_next_any<FMT, KIND, AL>(p, L, ph, R.f, kend, ok);
  }
}

template <int D, int AL>
__device__ __forceinline__ void ring_fill_acts(RingN<D>& R) {
#pragma unroll
  for (int d = 0; d < D; ++d) fetch_acts_n<AL>(R.f.ab, R.aop[d], R.r[d]);
}

// PEEL: the first round is its own copy, so that the loop's waits are
// counted from the steady load order (a split fill issues them in another).
// Up/gate (KIND 1): chunks are claimed from the CU's counter and chunk ends
// go through the partial windows.
template <int FMT, int KIND, bool PEEL, int D, int AL>
__device__ __forceinline__ void ring_run(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int k, int kend,
                                         int& jc, bool& ok) {
  EatN e;
  e.k = k;
  e.nch = 0;
  const bool any =
      KIND == 1 ? eat_next_up<FMT, AL>(p, L, ph, e, R.f.nch) : eat_next_n<FMT, KIND, AL>(p, L, ph, e, kend);
  if (any) {
    const int lg = (threadIdx.x & 63) >> 4;
    const int split = ph_split<KIND>(ph);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // The loop is left only after a whole round of D slots: once the last
    // job has ended, the rest of the round multiplies dead items and
    // refills with dead loads.  So every path to an item's wait has issued
    // the same D-1 items since (an exit in mid-round would make the
    // compiler's wait counting assume fewer and drain the ring).
    bool done = false;
    auto round = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (FMT == 0 || e.fmt == 0) eat_item_n<0, AL>(split, lg, R.r[d], acc);
        else eat_item_n<1, AL>(split, lg, R.r[d], acc);
        fetch_item_n<FMT, AL>(R.f, R.r[d]);
        fetch_adv_n<FMT>(R.f);
        if (R.f.left == 0) fetch_next_any<FMT, KIND, AL>(p, L, ph, R.f, kend, ok);
        if (!done) {
          e.left = uni(e.left) - 1;
          if (e.left == 0) {
            if (KIND == 1) up_job_end(p, L, e, acc, ph.nw, ok);
            else if (e.pst) lds_st128(L.pbuf + e.pidx, __builtin_bit_cast(u32x4, acc));
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            MOE_JSTAMP(p, jc);
            balance(L, ++jc);
            done = KIND == 1 ? !eat_next_up<FMT, AL>(p, L, ph, e, R.f.nch)
                             : !eat_next_n<FMT, KIND, AL>(p, L, ph, e, kend);
          }
        }
      }
    };
    if (PEEL) round();
    if (!done) {
      for (;;) {
        round();
        if (done) break;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the dead items' loads
  __builtin_amdgcn_s_setprio(0);
}


// Zeroes the narrow partial region (n floats).
__device__ inline void zero_partials(const Lds& L, size_t n) {
  for (size_t i = 4 * (size_t)threadIdx.x; i < n; i += 4 * kThreads) *(u32x4*)(L.pbuf + i) = u32x4{0u, 0u, 0u, 0u};
}

// out[r][h] = P_shared + sum_p w[r][p] * P[r][p], fp32 FMA chain in slot
// order, rounded to bf16 once.  Narrow: each product is first summed over
// the K-phases of its tile in order (sum_kphases: the sum a wide job-end
// reduction forms).
__device__ __forceinline__ float down_product(const Params& p, const Lds& L, int r, int slot, int hl) {
  if (!p.narrow) return L.pbuf[((size_t)r * (p.K + 1) + slot) * p.hs + hl];
  return L.pbuf[((size_t)r * (p.K + 1) + slot) * p.pitch + hl];  // summed by sum_kphases
}

// Narrow: each (row, slot, h) product is first summed over its K-phases
// (in order, into the K-phase 0 copy) by one thread per product, so the
// row's chain below reads one value per slot.  Whole workgroup; ends
// synchronised.
__device__ inline void sum_kphases(const Params& p, const Lds& L, const Sched& s) {
  const size_t kstride = (size_t)p.T * (p.K + 1) * p.pitch;
  const int n = p.T * (p.K + 1) * s.hc;
  for (int t = threadIdx.x; t < n; t += kThreads) {
    const int rs = t / s.hc, hl = t - rs * s.hc;  // rs = row * (K+1) + slot
    float* q = L.pbuf + (size_t)rs * p.pitch + hl;
    float v = 0.f;
    for (int kp = 0; kp < p.wpt; ++kp) v += q[kp * kstride];
    if (!isfinite(v)) set_err(p.err, kErrMid);
    q[0] = v;
  }
  __syncthreads();
}

// RES: a residual, when given, is added in fp32 after the chain, then
// rounded once (the residual add of the unfused layout, folded in).  The
// wide stream has a kernel of its own for it (kModeForwardRes), so that its
// residual-free kernel keeps its code.
template <bool RES>
__device__ inline void combine(const Params& p, const Lds& L, const Sched& s) {
  for (int t = threadIdx.x; t < p.T * s.hc; t += kThreads) {
    const int r = t / s.hc, hl = t - r * s.hc;
    const size_t o = (size_t)r * p.H + s.h0 + hl;
    const uint32_t res = RES && p.residual ? p.residual[o] : 0u;  // issued ahead of the chain
    float acc = p.n_shared ? down_product(p, L, r, p.K, hl) : 0.f;
    for (int k = 0; k < p.K; ++k) acc = fmaf(L.w[r * p.K + k], down_product(p, L, r, k, hl), acc);
    if (RES && p.residual) acc += bf16_bits_to_f32(res);
    p.out[o] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

// ------------------------------------------------------------------ kernel

__device__ __forceinline__ Sched make_sched(const Params& p, int G, int narrow) {
  Sched s;
  s.sh_tiles = p.n_shared ? p.Is / 8 : 0;
  s.rt_tiles = p.I / 8;
  s.G = G;
  s.n_jobs = s.sh_tiles + (G - p.n_shared) * s.rt_tiles;
  s.h0 = blockIdx.x * p.hs;
  s.hc = uni(p.H) - s.h0 < uni(p.hs) ? uni(p.H) - s.h0 : uni(p.hs);
  if (s.hc < 0) s.hc = 0;
  s.nrt = (s.hc + 15) / 16;
  s.nrt_p = uni(p.nrt_p);
  s.wpt = uni(p.wpt);
  s.narrow = narrow;
  return s;
}

// The kernel-argument block (the kernel's one argument, at offset 0 of the
// argument segment), through an opaque copy of its address: loads through
// it are not merged with loads before this point.  Used between the stages
// of the narrow path, so that argument values are loaded again where needed
// instead of being held in scalar registers across the weight stream.
typedef const __attribute__((address_space(4))) Params KArgs;
__device__ __forceinline__ const Params& fresh_args() {
  KArgs* q = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *(const Params*)q;
}

// The narrow forward after the logits: routing and grouping, the up/gate
// stream (its sums formed at job ends), the second flag barrier, the down
// stream, the combine.  With at most as many rows as waves, the waves that
// route no row start on this CU's shared-expert jobs once every row's
// scores are in, the routing waves but wave 7 as soon as their row is
// routed, and wave 7 once it has grouped the uses and written the routed
// tables.
template <int FMT, int AL>
__device__ __forceinline__ void narrow_forward(char* smem, uint32_t epoch) {
  const int wave = wave_id();
  int jn = 0;  // jobs this wave has ended (for balance)
  bool ok = true;
  {
    RingN<ring_up<AL>()> R;
    const Params& p = fresh_args();
    const Lds L = lds_map(smem, p);
    const int nkb = p.H / 128;
    PhaseN ph = {};
    ph.nw = nkb < kWaves ? nkb : kWaves;
    const int nS = shared_jobs_here(p);
    const bool early = p.T <= kWaves && p.T * p.K <= 64 && nS > 0;
    MOE_STAMP(p, 2);
    if (early) {
      // The top T waves route (row r by wave 7 - r; the scores of a batch
      // under 8 rows are published by wave 0), wave 7 then groups.  The
      // streaming waves start once every row's scores are in: their loads
      // would otherwise queue ahead of the polls.  The routing waves run at
      // raised priority until their rows are routed.
      const int r = kWaves - 1 - wave;
      if (r < p.T) {
        __builtin_amdgcn_s_setprio(3);
        route_row<true>(p, L, r, epoch + 1);
        if (r != 0) __builtin_amdgcn_s_setprio(0);
        lds_inc_lane0((uint32_t*)(L.misc + kMiscRouted));  // after this wave's ids / w writes (LDS order)
      }
      if (r == 0) {
        lds_wait<1>(p, (const uint32_t*)L.misc + kMiscRouted, (uint32_t)p.T, ok);
        MOE_LSTAMP(p, 10);
        groups_one_wave(p, L);
        wave_sync();
        MOE_LSTAMP(p, 3);
        const int G = lds_ldi_uniform(L.misc);
        const Sched s = make_sched(p, G, 1);
        const int nU = (int)blockIdx.x < s.n_jobs ? (s.n_jobs - 1 - (int)blockIdx.x) / p.ncu + 1 : 0;
        routed_tables<1>(p, L, s, nS, nU, threadIdx.x & 63, 64);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the up/gate tables, before the flag
        lds_st32(L.misc + kMiscReady, 1u);
        // the down tables are read after the phase barrier
        routed_tables<2>(p, L, s, nS, nU, threadIdx.x & 63, 64);
        __builtin_amdgcn_s_setprio(0);
        MOE_LSTAMP(p, 11);
      }
      if (r >= p.T) lds_wait<1>(p, (const uint32_t*)L.misc + kMiscPolled, (uint32_t)p.T, ok);
    } else {
      for (int r = wave; r < p.T; r += kWaves) route_row<true>(p, L, r, epoch + 1);
      __syncthreads();
      MOE_STAMP(p, 10);
      build_groups(p, L);
      MOE_STAMP(p, 3);
      const int G = lds_ldi_uniform(L.misc);
      const Sched s = make_sched(p, G, 1);
      const int nU = (int)blockIdx.x < s.n_jobs ? (s.n_jobs - 1 - (int)blockIdx.x) / p.ncu + 1 : 0;
      routed_tables(p, L, s, nS, nU, threadIdx.x, kThreads);
      if (threadIdx.x == 0) L.misc[kMiscReady] = 1;
      __syncthreads();
      MOE_STAMP(p, 11);
    }
    ring_open<FMT, 1, ring_up<AL>(), AL>(p, L, ph, R, 0, nS, ok);
    MOE_STAMP(p, 62);
    ring_fill<FMT, 1, false, ring_up<AL>(), AL>(p, L, ph, R, nS, ok);
    MOE_STAMP(p, 13);
    ring_run<FMT, 1, false, ring_up<AL>(), AL>(p, L, ph, R, 0, nS, jn, ok);
    MOE_WSTAMP(p, 0);
    MOE_TVAL(p, 8, jn);
  }
  int G;
  {
    const Params& p = fresh_args();
    const Lds L = lds_map(smem, p);
    MOE_STAMP(p, 4);
    publish(p, epoch + 2);
    MOE_STAMP(p, 12);
    G = lds_ldi_uniform(L.misc);
    const Sched s = make_sched(p, G, 1);
    zero_partials(L, (size_t)p.wpt * p.T * (p.K + 1) * p.pitch);
    // down: wave w takes tile w % nrt_p of this CU's slice and K-blocks
    // w / nrt_p + wpt*i of it
    PhaseN ph;
    ph.rt = wave % s.nrt_p;
    ph.k0 = wave / s.nrt_p;
    ph.lstep = 31 - __builtin_clz(s.wpt);
    ph.hb = s.h0 + 16 * ph.rt;
    ph.nlive = s.hc - 16 * ph.rt < 16 ? s.hc - 16 * ph.rt : 16;
    ph.split = (ph.hb / 128 + 1) * 128 - ph.hb;  // a 16-row tile spans at most two scale block rows
    ph.dnb = ph.nlive > 0 ? ((ph.hb + ph.nlive - 1) >> 7) - (ph.hb >> 7) : 0;
    ph.nw = 0;
    const int kend = ph.nlive > 0 ? p.qcap + s.G : p.qcap;
    // the first D items' weights do not depend on mid: issue them before the
    // wait, their activations after it
    RingN<kRingDD> R;
    ring_open<FMT, 2, kRingDD, AL>(p, L, ph, R, p.qcap, kend, ok);
    ring_fill<FMT, 2, true, kRingDD, AL>(p, L, ph, R, kend, ok);
    wait_all(p, epoch + 2);
    MOE_STAMP(p, 5);
    MOE_WSTAMP(p, 1);
    ring_fill_acts<kRingDD, AL>(R);
    ring_run<FMT, 2, true, kRingDD, AL>(p, L, ph, R, p.qcap, kend, jn, ok);
    MOE_WSTAMP(p, 2);
    MOE_STAMP(p, 6);
  }
  {
    const Params& p = fresh_args();
    const Lds L = lds_map(smem, p);
    const Sched s = make_sched(p, G, 1);
    __syncthreads();
    sum_kphases(p, L, s);
    combine<true>(p, L, s);
    MOE_STAMP(p, 7);
#ifdef MOE_TIMELINE
    __syncthreads();
    if (threadIdx.x < 64 && p.timeline) p.timeline[blockIdx.x * 64 + threadIdx.x] = MOE_TL(p, threadIdx.x);
#endif
  }
}


// NARROW = 1: the narrow stream (per-wave partials, 4 activation loads per
// item); 2 and 3: the same for batches of up to 4 and 8 rows (1 and 2
// loads per item, see lane_col); 0: the wide stream
// (up to four 16-column tiles per group, owner reductions).
template <int MODE, int FMT, int NARROW>
__global__ __launch_bounds__(kThreads, 1) void moe_fused(Params p) {
  constexpr int NPRE = NARROW ? 1 : 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Lds L = lds_map(smem, p);
  const int tid = threadIdx.x, wave = wave_id();

  MOE_STAMP(p, 0);
  constexpr bool kFwd = MODE == kModeForward || MODE == kModeForwardRes;
  if (NARROW && kFwd) {
    // Every wave reads the epoch for itself and first needs it to tag its
    // scores, after the router loads have come in.  The stream's LDS words
    // are set before the first meeting.  The scores are read through their
    // tags, so no flag is raised after them (waiting for the score stores
    // to reach memory would hold the workgroup for a store round trip).
    const uint32_t ep = __hip_atomic_load(&p.flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 64) L.ctl[tid] = 0u;
    stream_init(p, L, shared_jobs_here(p));
    __syncthreads();
    if (NARROW == 2 || p.T < kWaves) {  // (NARROW 2 runs at most 4 rows)
      router_logits(p, L, ep, 1u);
      // the logit partials lie in wave 0's routing scratch (wave 0 reads
      // them) unless the experts are few
      const int nd = (p.E > (int)blockIdx.x ? (p.E - 1 - (int)blockIdx.x) / p.ncu + 1 : 0) * p.T;
      if (kWaves * nd > p.E) __syncthreads();
    } else {
      router_logits_rows<true>(p, ep);
    }
    MOE_STAMP(p, 1);
    narrow_forward<FMT, NARROW == 2 ? 1 : NARROW == 3 ? 2 : 4>(smem, __builtin_amdgcn_readfirstlane(ep));
    return;
  }
  if (tid < 64) L.ctl[tid] = 0u;
  if (tid == 0)
    L.misc[1] = (int32_t)__hip_atomic_load(&p.flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t epoch = (uint32_t)__builtin_amdgcn_readfirstlane(L.misc[1]);

  // S0: router logits of this CU's experts, published for every CU
  if (NARROW && p.T < kWaves) router_logits(p, L, epoch, 1u);
  else router_logits_rows<false>(p, epoch + 1);
  publish(p, epoch + 1);
  MOE_STAMP(p, 1);
  if (!kFwd && blockIdx.x != 0) return;

  // S2 (wide stream, and the routing-only calls): route every row, then
  // group the step's distinct experts.  A wave of a narrow call has at most
  // two rows and polls their score slots; the wide stream waits for every
  // CU's flag first and reads them from L2.
  if (NARROW == 0) wait_all(p, epoch + 1);
  MOE_STAMP(p, 2);
  for (int r = wave; r < p.T; r += kWaves) route_row<NARROW != 0>(p, L, r, epoch + 1);
  __syncthreads();
  MOE_STAMP(p, 10);
  if (MODE == kModeRoute) {
    for (int u = tid; u < p.T * p.K; u += kThreads) {
      p.ids_out[u] = L.ids[u];
      p.w_out[u] = L.w[u];
    }
    return;
  }
  build_groups(p, L);
  MOE_STAMP(p, 3);
  const int G = __builtin_amdgcn_readfirstlane(L.misc[0]);
  if (MODE == kModeGroups) {
    int32_t* o = p.groups_out;
    if (tid == 0) {
      o[0] = G; o[1] = p.T; o[2] = p.K; o[3] = p.n_shared;
    }
    // g differs per thread here, so plain LDS reads
    for (int g = tid; g < G; g += kThreads) {
      o[4 + g] = p.n_shared && g == 0 ? -1 : L.gexp[g];
      o[4 + G + g] = p.n_shared && g == 0 ? p.T : L.gcnt[g];
      o[4 + 2 * G + g] = p.n_shared && g == 0 ? 0 : L.gstart[g];
    }
    const int ncol = p.T * (p.K + p.n_shared);
    for (int c = tid; c < ncol; c += kThreads) o[4 + 3 * G + c] = L.cols[c];
    return;
  }

  const Sched s = make_sched(p, G, 0);
  bool ok = true;
  int jc = 0;  // jobs ended
  Owned own;
  own.jc = -1;
  constexpr int MAXCT = max_tiles<NPRE>();
  f32x4 acc[MAXCT];
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  It up = It{0, first_job(p, 0), 0, 0, 0};
  settle(p, s, up);
  run_phase<NPRE, FMT>(p, L, s, up, 2, acc, jc, own, ok);
  MOE_WSTAMP(p, 0);

  It down = It{2, 0, 0, 0, 0};
  settle(p, s, down);
  MOE_STAMP(p, 4);
  service<NPRE>(p, L, own, true, ok);  // this wave's last owned up/gate job
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_st32(L.ctl + kCtlMidOut + wave, 1u);
  if (wave == 0) {
    lds_wait<8>(p, L.ctl + kCtlMidOut, 1u, ok);
    MOE_STAMP(p, 11);
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(&p.flags[blockIdx.x], epoch + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    MOE_STAMP(p, 12);
    if (down.phase == 2) poll_flags(p, epoch + 2);
    MOE_STAMP(p, 13);
    lds_st32(L.ctl + kCtlCrossed, 1u);
  }
  if (down.phase == 2) lds_wait<1>(p, L.ctl + kCtlCrossed, 1u, ok);
  MOE_STAMP(p, 5);
  MOE_WSTAMP(p, 1);

  run_phase<NPRE, FMT>(p, L, s, down, 3, acc, jc, own, ok);
  MOE_WSTAMP(p, 2);
  service<NPRE>(p, L, own, true, ok);  // the last owned down job
  MOE_STAMP(p, 6);
  __syncthreads();

  // S5: combine this CU's output rows
  combine<MODE == kModeForwardRes>(p, L, s);
  MOE_STAMP(p, 7);
#ifdef MOE_TIMELINE
  __syncthreads();
  if (tid < 64 && p.timeline) p.timeline[blockIdx.x * 64 + tid] = MOE_TL(p, tid);
#endif
}

// ------------------------------------------------------------------ host glue

#ifndef MOE_RES_WIDE_TU
WsLayout ws_layout(int max_rows, int E, int K, int H, int I, int Is) {
  (void)H;
  WsLayout w;
  size_t q = 0;
  w.flags = q; q = align_up(q + 4 * 1024, 256);
  w.err = q; q = align_up(q + 256, 256);
  w.scores = q; q = align_up(q + 16 * (size_t)max_rows * E, 256);
  w.mid_ld = (I > Is ? I : Is);
  w.mid = q; q = align_up(q + 2 * (size_t)max_rows * (K + 1) * w.mid_ld, 256);
  w.total = q;
  return w;
}

#endif

// Per kernel instance and device: the largest LDS size for which the
// instance's dynamic LDS limit has been raised and one workgroup of kThreads
// was found to fit on a CU (so the grid of one workgroup per CU can be
// resident at once on an otherwise idle device).  Checked once per size
// increase; later calls launch at once.
static bool resident_ok(const void* kfn, std::atomic<int>& ok_lds, int lds, hipError_t& e) {
  e = hipSuccess;
  int have = ok_lds.load(std::memory_order_acquire);
  if (lds <= have) return true;
  e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return false;
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kfn, kThreads, (size_t)lds);
  if (e != hipSuccess) return false;
  if (nb < 1) {
    e = hipErrorCooperativeLaunchTooLarge;
    return false;
  }
  while (have < lds && !ok_lds.compare_exchange_weak(have, lds, std::memory_order_acq_rel)) {
  }
  return true;
}

template <int MODE, int FMT, int NARROW = 1>
static hipError_t launch_one(const Params& p, hipStream_t stream, int dev) {
  static std::atomic<int> ok_lds[kMaxDevices];
  auto kfn = moe_fused<MODE, FMT, NARROW>;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipError_t e;
  if (!resident_ok((const void*)kfn, ok_lds[dev], p.lds_bytes, e)) return e;
  hipLaunchKernelGGL(kfn, dim3(p.ncu), dim3(kThreads), p.lds_bytes, stream, p);
  return hipGetLastError();
}

#ifndef MOE_RES_WIDE_TU
hipError_t launch(const Params& p, int mode, hipStream_t stream, int dev) {
  const bool wide = !p.narrow;
  const int nk = p.T <= 4 ? 2 : p.T <= 8 ? 3 : 1;  // narrow kernel by batch size
  const bool wide_res = mode == kModeForward && wide && p.residual;
  if (p.routed_fmt == 0 && !wide_res) {
    if (mode == kModeForward)
      return wide      ? launch_one<kModeForward, 0, 0>(p, stream, dev)
             : nk == 2 ? launch_one<kModeForward, 0, 2>(p, stream, dev)
             : nk == 3 ? launch_one<kModeForward, 0, 3>(p, stream, dev)
                       : launch_one<kModeForward, 0, 1>(p, stream, dev);
    if (mode == kModeRoute) return launch_one<kModeRoute, 0>(p, stream, dev);
    return launch_one<kModeGroups, 0>(p, stream, dev);
  }
  if (!wide_res) {
    if (mode == kModeForward)
      return wide      ? launch_one<kModeForward, 1, 0>(p, stream, dev)
             : nk == 2 ? launch_one<kModeForward, 1, 2>(p, stream, dev)
             : nk == 3 ? launch_one<kModeForward, 1, 3>(p, stream, dev)
                       : launch_one<kModeForward, 1, 1>(p, stream, dev);
    if (mode == kModeRoute) return launch_one<kModeRoute, 1>(p, stream, dev);
    return launch_one<kModeGroups, 1>(p, stream, dev);
  }
  return launch_res_wide(p, stream, dev);
}
#else
// The wide stream with a residual: its kernels are built in a translation
// unit of their own (moe_kernels_res.hip), so that the code object of the
// other kernels is the same with or without them.
hipError_t launch_res_wide(const Params& p, hipStream_t stream, int dev) {
  return p.routed_fmt == 0 ? launch_one<kModeForwardRes, 0, 0>(p, stream, dev)
                           : launch_one<kModeForwardRes, 1, 0>(p, stream, dev);
}
#endif

}  // namespace moe
