// moe_kernels.hip -- the fused decode MoE pass for MI355X (gfx950, CDNA4).
//
// One persistent launch: one workgroup of 8 waves per CU, all resident.
//
//   S0  router logits   l[r][e] for a block of (row, expert) dots per CU
//                       (fp64 sums of exact bf16 products, one summation
//                       order at every batch size) and sigmoid; each score
//                       goes to a slot tagged with the call's epoch, so no
//                       flag barrier is needed.
//   S1  shared up/gate  the shared expert does not depend on routing, so its
//                       tiles are streamed while the routing runs.
//   S2  route + group   below 8 rows every CU polls the score slots of every
//                       row until they carry the call's tag and routes every
//                       row itself (no hand-off); from 8 rows each row is
//                       routed by one CU, which publishes the row's picks as
//                       tagged words that every CU polls.  Each CU then
//                       builds the step's group table in LDS: distinct
//                       experts in order of first use, found by ballot /
//                       prefix count, each with its using rows.
//   S3  routed up/gate  jobs (group, tile of 8 or 16 intermediates) dealt
//                       round-robin over CUs; each job streams its gate and
//                       up weight rows once and uses every row of the group
//                       as an MFMA column; SwiGLU mid values go to the
//                       workspace.
//   S4  down            after the one flag barrier of the call (the
//                       meeting), CU c owns output rows [c*hs, (c+1)*hs) and
//                       streams that slice of every used expert's W_down
//                       once; per (row, slot) products stay in LDS.  Unit
//                       batches that lie past the step's groups issue
//                       nothing (dead-batch skip).
//   S5  combine         out[r][h] = shared + sum_p w[r][p] * P[r][p][h] in this
//                       row-local order, rounded to bf16 once (under an expert
//                       range, p over the picks whose expert is held here).
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
// Cross-CU data (scores, picks, mid) is stored at agent scope (written
// through to the device's point of coherence), so raising a flag after it
// needs only the workgroup's own store completion, not an L2 writeback.
// Readers poll the flags (or, for scores and picks, the epoch tags in the
// words themselves) and then acquire at agent scope.  Each CU owns one
// flag; a call advances every flag by two (the forward raises it straight
// to epoch + 2 at the meeting, the routing-only calls to epoch + 1), so the
// workspace needs no reset.  Waits are bounded:
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
    if (threadIdx.x == 0 && (p).timeline && (jc) < 12)                                   \
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
  int32_t* misc;     // [32]: 0 = G, 1 = epoch, 8.. = scan, kMisc* words
  uint32_t* ctl;     // [64] stream counters (see kCtl*)
  double* rb;        // [kWaves][E] router keys (routing scratch, see lds_offsets)
  double* rgs;       // [kWaves][64] group scores
  int32_t* rkept;    // [kWaves][64]
  double* rcb;       // [kWaves][E] top-k candidates: key b
  double* rcs;       // [kWaves][E] and score s
  int32_t* rce;      // [kWaves][E] and expert
  float* pbuf;       // the per-wave partials (see lds_offsets)
  struct JobDesc* jd;  // job descriptors (this CU's up/gate jobs, then the down jobs)
  uint32_t* wcnt;    // [kPuWin] chunks of the job in each partial window that have ended
  uint32_t* wgen;    // [kPuWin] jobs summed out of each window
  uint32_t* ccnt;    // up/gate chunks claimed by this CU's waves ([1]: down jobs claimed)
  uint32_t* cfifo;   // [kWaves][8] each wave's claimed chunks, fetch side to multiplying side
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// LDS words of the stream's start (misc[]).
constexpr int kMiscNU = 2;      // this CU's up/gate jobs, once routed
constexpr int kMiscReady = 3;   // 1 once the routed jobs' tables are written
constexpr int kMiscRouted = 4;  // rows routed so far (early start)
constexpr int kMiscPolled = 5;  // rows whose scores are in (early start)
constexpr int kMiscND = 6;      // down job entries (groups x column tiles), once routed

// Every wave keeps its partial tiles apart in LDS, and they are summed over
// the waves in wave order:
//   up/gate  Pu[win][w][col][2*ti], win = local job mod kPuWin (w = 0..7,
//            the job's K-phase; col < pcols, the job's column; ti gate rows
//            then ti up rows), summed by the wave that ends the job's last
//            chunk
//   down     Pd[kp][row][slot][pitch]  (kp = 0..wpt-1, the K-phase of the
//            waves that share a 16-row down tile; h along the slice),
//            summed in the combine; with wpt = 1 (above kKsplitRows rows)
//            each down job is one wave's whole sum
// Pu and Pd share one region (Pu is done with before Pd is written), which
// also holds the routing scratch before the stream, except in a call of at
// most as many rows as waves, whose waves stream while other rows are
// routed.  The job descriptors (qcap up/gate entries, then dcap down
// entries) sit before it.
constexpr int kPuWin = 8;
struct LdsOffsets {
  size_t ids, w, first, egrp, rmask, gexp, gcnt, gstart, cols, cgrp, misc, ctl, wst, jd, rs, pbuf, total;
};
constexpr size_t kJobDescBytes = 48;

__host__ __device__ inline LdsOffsets lds_offsets(const Params& p) {
  LdsOffsets o;
#ifdef MOE_TIMELINE
  size_t q = 64 * 8;  // the stamps first (see MOE_TL)
#else
  size_t q = 0;
#endif
  const int T = p.T, K = p.K, E = p.E;
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
  o.jd = q; q = align_up(q + kJobDescBytes * (size_t)(p.qcap + p.dcap), 16);
  // routing scratch: rb, rgs, rkept, then the top-k candidates (b, s, e),
  // one slot per wave that routes at once
  o.rs = q;
  const size_t ns = (size_t)p.rslots;
  const size_t rs = 8 * ns * E + 8 * ns * 64 + 4 * ns * 64 + 20 * ns * E;
  const size_t pu = 4 * (size_t)kPuWin * kWaves * p.pcols * 2 * p.ti;
  const size_t pd = 4 * (size_t)p.wpt * T * (K + 1) * p.pitch;
  const size_t need = pu > pd ? pu : pd;
  size_t end;
  if (!p.rsover) {
    o.pbuf = align_up(q + rs, 16);
    end = o.pbuf + need;
  } else {
    o.pbuf = q;
    end = q + (need > rs ? need : rs);
  }
  o.total = align_up(end, 16);
  return o;
}

// Bounds of the job tables.  Up/gate: a CU gets at most ceil(tiles/ncu)
// tiles of each group, and a group of c columns is ceil(c/cpj) jobs per tile;
// over a batch the routed groups number at most min(E, T*K) with T*K
// columns, so their column tiles number at most min(E, T*K) + T*K/cpj.
size_t stream_geometry(Params& p, bool fp8_tiles) {
  const int nrt = (p.hs + 15) / 16;
  p.nrt_p = nrt <= 1 ? 1 : nrt <= 2 ? 2 : 4;
  p.kph = kWaves / p.nrt_p;
  p.wpt = p.T <= kKsplitRows ? p.kph : 1;
  p.pitch = 16 * nrt;
  p.cpj = 4 * stream_al(p.T);
  p.pcols = p.T < p.cpj ? p.T : p.cpj;
  p.ti = stream_ti(p.T, fp8_tiles ? 0 : p.routed_fmt);
  if (p.ti == 16 && (fp8_tiles || p.routed_fmt == 0)) {
    // FP8 two-tile items only where a CU has many (group, tile) pairs: with
    // few (an expert range of 32 experts) the coarser jobs end unevenly
    const int groups = (p.ec < p.T * p.K ? p.ec : p.T * p.K) + p.n_shared;
    if ((long)groups * (p.I / 16) < 32L * p.ncu) p.ti = 8;
  }
  p.lti = p.ti == 16 ? 4 : 3;
  const int tk = p.T * p.K;
  const int nct_sh = p.n_shared ? (p.T + p.cpj - 1) / p.cpj : 0;
  const int ct_routed = (p.E < tk ? p.E : tk) + (tk + p.cpj - 1) / p.cpj;
  const int sh_tiles = p.n_shared ? p.Is >> p.lti : 0, rt_tiles = p.I >> p.lti;
  const int per_sh = (sh_tiles + p.ncu - 1) / p.ncu, per_rt = (rt_tiles + p.ncu - 1) / p.ncu;
  p.qcap = per_sh * nct_sh + per_rt * ct_routed;
  p.dcap = nct_sh + ct_routed;
  return lds_offsets(p).total;
}

__device__ inline Lds lds_map(char* base, const Params& p) {
  LdsOffsets o = lds_offsets(p);
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
  L.pbuf = (float*)(base + o.pbuf);
  const size_t ns = (size_t)p.rslots;
  L.rb = (double*)(base + o.rs);
  L.rgs = L.rb + ns * p.E;
  L.rkept = (int32_t*)(L.rgs + ns * 64);
  L.rcb = (double*)(L.rkept + ns * 64);
  L.rcs = L.rcb + ns * p.E;
  L.rce = (int32_t*)(L.rcs + ns * p.E);
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
// A row's slots are stored transposed by fours: expert e at
// (e mod 4) * E4 + e / 4 (E4 = E rounded up to 4, over 4), so the routing
// wave, whose lane l holds experts 4l..4l+3, reads one contiguous run of
// slots per load instruction.
__device__ __forceinline__ int slot_e4(int E) { return (E + 3) >> 2; }
__device__ __forceinline__ size_t score_slot(const Params& p, int r, int e) {
  const int e4 = slot_e4(p.E);
  return (size_t)r * 4 * e4 + (size_t)(e & 3) * e4 + (e >> 2);
}
__device__ __forceinline__ void publish_score(const Params& p, int r, int e, double s, uint32_t tag) {
  uint64_t* dst = (uint64_t*)p.scores + score_slot(p, r, e) * 2;
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
// tree (wave_sum_d), and the chunk sums are added in chunk order.  Used from
// 8 rows up.  The T x E dots are cut into blocks of rb rows by eb experts,
// one block per CU, with rb and eb near the square root of a CU's share:
// every CU reads rb rows of x and eb router rows (not every row of x, which
// at 64 rows made the logits bound by the L2's bandwidth); at 8 rows the
// block is one expert's column.  Wave w takes the
// block's dots w, w + 8, ... (row-fastest); when the block's row count
// divides 8 a wave keeps one row, whose x it loads once.
// LATE: `v` is the epoch, a load still in flight, first read once the sums
// are formed (tag = epoch + 1); otherwise `v` is the tag.
template <bool LATE>
__device__ inline void router_logits_rows(const Params& p, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= kWaves) return;
  const int ch = p.H / kWaves, ngrp = ch >> 3;
  const int g0 = lane < ngrp ? lane : ngrp - 1, g1 = lane + 64 < ngrp ? lane + 64 : g0;
  // row blocks (a power of two; pe = ncu / pr expert blocks).  Up to 8
  // rows one block row: CU c takes expert c and wave w row w, so the rows
  // of the fast waves (the older wave of each SIMD) are complete early and
  // their routing overlaps the wait for the others.
  int pr = 1;
  while (p.T > kWaves && pr < p.T && 2 * pr <= p.ncu && 4 * pr * pr * p.E <= p.T * p.ncu) pr *= 2;
  while ((p.T + pr - 1) / pr > kWaves && 2 * pr <= p.ncu) pr *= 2;
  const int pe = p.ncu / pr;
  const int rb = (p.T + pr - 1) / pr, eb = (p.E + pe - 1) / pe;
  const int c = (int)blockIdx.x;
  if (c >= pr * pe) return;
  const int r0 = (c / pe) * rb, e0 = (c % pe) * eb;
  const int nr = p.T - r0 < rb ? p.T - r0 : rb, ne = p.E - e0 < eb ? p.E - e0 : eb;
  if (nr <= 0 || ne <= 0) return;
  u32x4 xv[kWaves][2];
  int xrow = -1;
  for (int d = wave; d < nr * ne; d += kWaves) {
    const int r = r0 + d % nr, e = e0 + d / nr;
    if (r != xrow) {
      const uint16_t* xr = p.x + (size_t)r * p.H;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        xv[k][0] = ld16(xr + (size_t)k * ch + 8 * g0);
        xv[k][1] = ld16(xr + (size_t)k * ch + 8 * g1);
      }
      xrow = r;
    }
    const uint16_t* wr = p.router_w + (size_t)e * p.H;
    u32x4 wv[kWaves][2];
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      wv[k][0] = ld16(wr + (size_t)k * ch + 8 * g0);
      wv[k][1] = ld16(wr + (size_t)k * ch + 8 * g1);
    }
    // LATE: the bias bits are converted once the sums are formed
    const uint32_t braw = LATE ? load_bias_raw(p, e) : 0u;
    const double bias = LATE ? 0.0 : load_bias(p, e);
    double l = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      double acc = 0.0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q == 0 ? lane < ngrp : lane + 64 < ngrp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t xa = xv[k][q][i], wa = wv[k][q][i];
            acc = fma((double)bf16_bits_to_f32(xa & 0xffffu), (double)bf16_bits_to_f32(wa & 0xffffu), acc);
            acc = fma((double)bf16_bits_to_f32(xa >> 16), (double)bf16_bits_to_f32(wa >> 16), acc);
          }
        }
      }
      l += wave_sum_d(acc);
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

// The row whose routing the timeline build stamps: row 0, or above 8 rows
// (one row per routing CU) this CU's own row.
__device__ __forceinline__ int tl_row(const Params& p) { return p.T > kWaves ? (int)blockIdx.x : 0; }

// Two largest values (t1 >= t2) over an aligned lane group, one exchange
// step: the larger of the two firsts, and the larger of the smaller first
// and the two seconds.
template <int CTRL>
__device__ __forceinline__ void top2_step(double& t1, double& t2) {
  const double o1 = xlane_d<CTRL>(t1), o2 = xlane_d<CTRL>(t2);
  const double hi = fmax(t1, o1), lo = fmin(t1, o1);
  t2 = fmax(lo, fmax(t2, o2));
  t1 = hi;
}

// Routes row r with one wave: group stage (sum of the two best keys per
// group, keep k_g groups by (score desc, index asc)), then the top K by
// (key desc, index asc); weights s/sum(s)*scale in fp64.
// Lane l holds experts 4l .. 4l+3, so a group of 4m experts (m a power of
// two) is an aligned run of m lanes.
// Polls row r's score slots (agent-scope loads) until every one carries
// this call's tag (bounded: on timeout the error bit is set and routing
// runs on).  `slot`: the wave's part of the routing scratch (waves that
// route at the same time use different slots).
__device__ inline void route_row(const Params& p, const Lds& L, int r, uint32_t tag, int slot) {
  const int lane = threadIdx.x & 63;
  typedef __attribute__((address_space(1))) uint64_t G64;
  const G64* sc = (const G64*)p.scores + score_slot(p, r, 0) * 2;  // the row's first slot
  const int e4 = slot_e4(p.E);
  uint64_t w0[4] = {0, 0, 0, 0}, w1[4] = {0, 0, 0, 0};
  double bias[4];  // loaded first: they do not depend on the scores
#pragma unroll
  for (int i = 0; i < 4; ++i) bias[i] = 4 * lane + i < p.E ? load_bias(p, 4 * lane + i) : 0.0;
  // a slot is loaded again only until both its words carry the tag, so the
  // later rounds of the poll fetch only the slots still missing
  bool got[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) got[i] = 4 * lane + i >= p.E;
  for (int spins = 0;;) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = i * e4 + lane;  // q: expert 4 * lane + i's slot in the row
      if (!got[i]) {
        w0[i] = __hip_atomic_load(sc + 2 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w1[i] = __hip_atomic_load(sc + 2 * q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        got[i] = (uint32_t)(w0[i] >> 32) == tag && (uint32_t)(w1[i] >> 32) == tag;
      }
      ready = ready && got[i];
    }
    if (__all(ready)) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) set_err(p.err, kErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (r == tl_row(p)) MOE_LSTAMP(p, 9);
  if (lane == 0)  // rows whose scores are in (see narrow_forward)
    __hip_atomic_fetch_add((__attribute__((address_space(3))) uint32_t*)(L.misc + kMiscPolled), 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  double bv[4], sv[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    alive[i] = e < p.E;
    const double s = __builtin_bit_cast(double, (w0[i] << 32) | (w1[i] & 0xffffffffull));
    const double b = alive[i] ? s + bias[i] : -INFINITY;
    sv[i] = alive[i] ? s : 0.0;
    bv[i] = isnan(b) ? -INFINITY : b;
  }
  if (r == tl_row(p)) MOE_LSTAMP(p, 60);
  if (p.ng > 1) {
    const int gsz = p.E / p.ng, lpg = gsz >> 2;
    if ((gsz & 3) == 0 && lpg <= 64 && (lpg & (lpg - 1)) == 0) {
      // the lane's own two best keys, then a butterfly over the group's lanes
      double t1 = fmax(bv[0], bv[1]), t2 = fmin(bv[0], bv[1]);
#pragma unroll
      for (int i = 2; i < 4; ++i) {
        t2 = fmax(t2, fmin(t1, bv[i]));
        t1 = fmax(t1, bv[i]);
      }
      if (lpg > 1) top2_step<kDppXor1>(t1, t2);
      if (lpg > 2) top2_step<kDppXor2>(t1, t2);
      if (lpg > 4) top2_step<kDppHalfMirror>(t1, t2);
      if (lpg > 8) top2_step<kDppMirror>(t1, t2);
      if (lpg > 16) top2_step<kSwizzleXor16>(t1, t2);
      if (lpg > 32) {
        const double o1 = __shfl_xor(t1, 32, 64), o2 = __shfl_xor(t2, 32, 64);
        const double hi = fmax(t1, o1), lo = fmin(t1, o1);
        t2 = fmax(lo, fmax(t2, o2));
        t1 = hi;
      }
      // rank of this lane's group (lane / lpg) among all groups, from each
      // group's score in its first lane
      const double gs = t1 + t2;
      const int own = lane / lpg;
      int rank = 0;
      for (int j = 0; j < p.ng; ++j) rank += key_before(readlane_d(gs, j * lpg), j, gs, own) ? 1 : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) alive[i] = alive[i] && rank < p.kg;
    } else {
      double* rb = L.rb + (size_t)slot * p.E;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (alive[i]) rb[4 * lane + i] = bv[i];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < p.ng) {
        double t1 = -INFINITY, t2 = -INFINITY;
        for (int e = lane * gsz; e < (lane + 1) * gsz; ++e) {
          double v = rb[e];
          if (v > t1) { t2 = t1; t1 = v; }
          else if (v > t2) { t2 = v; }
        }
        L.rgs[slot * 64 + lane] = t1 + t2;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < p.ng) {
        const double mine = L.rgs[slot * 64 + lane];
        int rank = 0;
        for (int j = 0; j < p.ng; ++j) rank += key_before(L.rgs[slot * 64 + j], j, mine, lane) ? 1 : 0;
        L.rkept[slot * 64 + lane] = rank < p.kg;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (alive[i]) alive[i] = L.rkept[slot * 64 + (4 * lane + i) / gsz] != 0;
    }
  }
  if (r == tl_row(p)) MOE_LSTAMP(p, 14);
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
  if (r == tl_row(p)) MOE_LSTAMP(p, 56);
  // (2) The candidates go to LDS in expert order; each is ranked exactly
  // by (b desc, e asc) against all of them.
  double* cb = L.rcb + (size_t)slot * p.E;
  double* cs = L.rcs + (size_t)slot * p.E;
  int32_t* ce = L.rce + (size_t)slot * p.E;
  int nc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool c = alive[i] && ord32((float)bv[i]) >= t;
    const unsigned long long bal = __ballot(c);
    if (c) {
      const int pos = nc + __popcll(bal & ((1ull << lane) - 1ull));
      cb[pos] = bv[i];
      cs[pos] = sv[i];
      ce[pos] = 4 * lane + i;
    }
    nc += __popcll(bal);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (r == tl_row(p)) MOE_LSTAMP(p, 57);
  double* ps = L.rgs + (size_t)slot * 64;  // the winners' s in pick order
  if (nc <= 8) {
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
  if (r == tl_row(p)) MOE_LSTAMP(p, 15);
  // every lane forms the same sum in pick order; lane k writes weight k
  double ssum = 0.0;
  for (int k = 0; k < p.K; ++k) ssum += ps[k];
  if (lane < p.K) L.w[r * p.K + lane] = (float)(ps[lane] / ssum * p.routed_scale);
  if (r == tl_row(p)) MOE_LSTAMP(p, 58);
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

// Inclusive prefix sum over the wave by DPP: running sums within each row
// of 16 lanes (shifts 1, 2, 4, 8, lanes shifted in from outside the row
// adding 0), then the row totals carried on by the row broadcasts of lanes
// 15 and 31.  No LDS round trip (a shuffle would be one per step).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
  return v;
}

// gstart[g] = base + sum of gcnt over groups g0..g-1, for g0 <= g < G, by
// one wave (64 groups per pass).
__device__ inline void scan_gstart(const Lds& L, int g0, int G, int base) {
  const int lane = threadIdx.x & 63;
  for (int c0 = g0; c0 < G; c0 += 64) {
    const int g = c0 + lane;
    const int c = g < G ? L.gcnt[g] : 0;
    const int v = wave_incl_scan(c);
    if (g < G) L.gstart[g] = base + v - c;
    base += __builtin_amdgcn_readlane(v, 63);
  }
}

// Column of use u = r*K + slot within its group: the rows using an expert,
// in ascending order (a row picks an expert at most once).
__device__ __forceinline__ int use_rank(const Lds& L, int e, int r) {
  const uint32_t lo = L.rmask[2 * e], hi = L.rmask[2 * e + 1];
  return r < 32 ? __popc(lo & ((1u << r) - 1u)) : __popc(lo) + __popc(hi & ((1u << (r - 32)) - 1u));
}

// Whether routed expert e is held here (the expert range of the config).
__device__ __forceinline__ bool held(const Params& p, int e) { return (unsigned)(e - p.ef) < (unsigned)p.ec; }

// Above 8 rows the rows are routed across CUs instead of every CU routing
// every row (eight rows or more per wave, one after another): row r by
// wave r / ncu of CU r mod ncu, which publishes the row's picks as tagged
// words (like the score slots); then every thread of every CU polls the
// picks of one use (row, slot) until both its words carry the call's tag.
// The routing arithmetic is the same whichever CU runs it, so the picks
// are the same bits as when every CU routes every row.
// Routes row r with the calling wave (routing scratch `slot`) and publishes
// its picks (lanes < K).
__device__ inline void route_publish(const Params& p, const Lds& L, int r, uint32_t tag, int slot) {
  const int lane = threadIdx.x & 63;
  typedef __attribute__((address_space(1))) uint64_t G64;
  route_row(p, L, r, tag, slot);
  wave_sync();  // the row's ids and weights, written by single lanes
  if (lane < p.K) {
    const uint32_t id = (uint32_t)L.ids[r * p.K + lane];
    const uint32_t wb = __float_as_uint(L.w[r * p.K + lane]);
    G64* q = (G64*)p.picks + 2 * (r * p.K + lane);
    __hip_atomic_store(q, ((uint64_t)tag << 32) | id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, ((uint64_t)tag << 32) | wb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  MOE_LSTAMP(p, 61);
}

// Reads the picks of uses u0, u0 + step, ... < T*K (at most PER per lane)
// into L.ids / L.w, polling them together (one round trip per round, the
// later rounds reloading only the uses still missing) until both words of
// each carry the call's tag.
template <int PER>
__device__ inline void read_picks(const Params& p, const Lds& L, uint32_t tag, int u0, int step) {
  typedef __attribute__((address_space(1))) uint64_t G64;
  constexpr int kPer = PER;
  const int U = p.T * p.K;
  uint64_t a[kPer], b[kPer];
  bool got[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    got[i] = u0 + i * step >= U;
    a[i] = 0;
    b[i] = 0;
  }
  for (int spins = 0;;) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!got[i]) {
        const G64* q = (const G64*)p.picks + 2 * (u0 + i * step);
        a[i] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        b[i] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!got[i]) got[i] = (uint32_t)(a[i] >> 32) == tag && (uint32_t)(b[i] >> 32) == tag;
      all = all && got[i];
    }
    if (__all(all)) break;
    if (++spins > kSpinLimit) {
      set_err(p.err, kErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = u0 + i * step;
    if (u < U) {
      L.ids[u] = (int32_t)(uint32_t)a[i];
      L.w[u] = __uint_as_float((uint32_t)b[i]);
    }
  }
}

__device__ inline void route_rows_spread(const Params& p, const Lds& L, uint32_t tag) {
  const int wave = threadIdx.x >> 6;
  for (int r = (int)blockIdx.x + wave * p.ncu; r < p.T; r += kWaves * p.ncu) route_publish(p, L, r, tag, wave);
  read_picks<kMaxRows * kMaxTopK / kThreads>(p, L, tag, (int)threadIdx.x, kThreads);
  MOE_STAMP(p, 63);
}

// The grouping by one wave (the narrow stream's wave 7) of up to 64 * PER
// uses, lane l taking uses l + 64 i, no workgroup barriers; the PER passes
// of each step are unrolled so that their LDS accesses overlap.  Uses of
// experts not held here form no group and get no column.
template <int PER>
__device__ inline void groups_one_wave(const Params& p, const Lds& L) {
  const int lane = threadIdx.x & 63;
  const int U = p.T * p.K;
  int ev[PER], rv[PER];
  bool hv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int u = lane + 64 * i;
    ev[i] = u < U ? L.ids[u] : 0;
    rv[i] = u / p.K;
    hv[i] = u < U && held(p, ev[i]);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (hv[i]) {
      L.first[ev[i]] = 0xffffffffu;
      L.rmask[2 * ev[i]] = 0u;
      L.rmask[2 * ev[i] + 1] = 0u;
    }
  }
  wave_sync();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (hv[i]) {
      atomicMin(&L.first[ev[i]], (uint32_t)(lane + 64 * i));
      atomicOr(&L.rmask[2 * ev[i] + (rv[i] >> 5)], 1u << (rv[i] & 31));
    }
  }
  wave_sync();
  // groups in order of first use
  uint32_t fv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) fv[i] = hv[i] ? L.first[ev[i]] : 0u;
  int G = p.n_shared;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool isf = hv[i] && fv[i] == (uint32_t)(lane + 64 * i);
    const unsigned long long m = __ballot(isf);
    if (isf) {
      const int g = G + __popcll(m & ((1ull << lane) - 1ull));
      const int e = ev[i];
      L.egrp[e] = g;
      L.gexp[g] = e;
      L.gcnt[g] = __popc(L.rmask[2 * e]) + __popc(L.rmask[2 * e + 1]);
    }
    G += __popcll(m);
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
  if (p.n_shared)
    for (int r = lane; r < p.T; r += 64) {
      L.cols[r] = r * 16 + p.K;
      L.cgrp[r] = 0;
    }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (hv[i]) {
      const int e = ev[i], r = rv[i];
      const int g = L.egrp[e], c = L.gstart[g] + use_rank(L, e, r);
      L.cols[c] = r * 16 + (lane + 64 * i - r * p.K);
      L.cgrp[c] = g;
    }
  }
}

__device__ inline void build_groups(const Params& p, const Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = p.T * p.K;
  if (U <= 64) {
    if (wave == 0) groups_one_wave<1>(p, L);
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
    if (!held(p, e)) continue;
    atomicMin(&L.first[e], (uint32_t)u);
    atomicOr(&L.rmask[2 * e + (r >> 5)], 1u << (r & 31));
  }
  __syncthreads();
  // exclusive prefix count of first uses, 512 uses per pass
  int base = p.n_shared;
  for (int u0 = 0; u0 < U; u0 += kThreads) {
    const int u = u0 + tid;
    const bool isf = u < U && held(p, L.ids[u]) && L.first[L.ids[u]] == (uint32_t)u;
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
    if (!held(p, e)) continue;
    const int g = L.egrp[e], c = L.gstart[g] + use_rank(L, e, r);
    L.cols[c] = r * 16 + slot;
    L.cgrp[c] = g;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ weight stream
//
// Each CU walks a sequence of jobs: its shared-expert up/gate tiles, its
// routed up/gate tiles (8 gate rows and their 8 up rows, or 16 and 16 in
// two-tile items, over all of H), then its down rows of every used expert
// (over that expert's intermediate size).  The 8 waves split every job
// along the reduction axis in K-phases: phase w holds the K-blocks w, w+8,
// w+16, ... (128 bytes of every weight row: 128 FP8 or 256 MXFP4 values).
// One K-block of one job is an item: the weights of one or two 16-row MFMA
// tiles (32 bytes per lane each), their block scales and the activations of
// the job's columns, shared by the tiles.  A wave loads its items
// straight from HBM into registers, D items ahead of the one it
// multiplies; every item issues the same number of loads, so the in-order
// wait for item n leaves items n+1..n+D-1 in flight.  (An LDS ring fed by
// LDS-DMA reached a lower and less steady share of HBM bandwidth.)


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

struct Sched {
  int sh_tiles;  // shared up/gate tiles (I_s / ti)
  int rt_tiles;  // routed up/gate tiles per group (I / ti)
  int n_pairs;   // all (group, tile) pairs, known after routing
  int G;         // groups, known after routing
  int h0, hc;    // this CU's down rows
  int nrt;       // 16-row tiles of them
  int nrt_p, wpt;  // tiles rounded up to 1, 2 or 4; copies of the down products
  int kph;         // K-phases of a down sum
};

__device__ __forceinline__ bool shared_group(const Params& p, int g) { return p.n_shared && g == 0; }

// Activation offset (elements) of column code `code` for lane group lg:
// x rows for up/gate, mid lines for down.
__device__ __forceinline__ uint32_t act_offset(const Params& p, int kind, int code, int lg) {
  const uint32_t t = kind == 1 ? lmul((uint32_t)(code >> 4), (uint32_t)p.H)
                               : lmul(lmul((uint32_t)(code >> 4), (uint32_t)(p.K + 1)) + (uint32_t)(code & 15),
                                      (uint32_t)p.mid_ld);
  return t + 32u * (uint32_t)lg;
}

// mid = silu(gate) * up in fp32 (one expression for both layouts).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

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

// ------------------------------------------------------------------ narrow stream
//
// Every batch size (the name is older than the wide batches): a group's
// columns go to jobs of at most 4 * AL columns (a column spans 4 / AL of
// the 16 MFMA columns), a group with more columns being several jobs.  A
// wave's
// items run through a D-deep register ring: each step multiplies the oldest
// item, refills its slot with the item D later and counts; only a job
// change on either side does more.  At a job end the wave stores its
// partial tile into its own part of LDS and never waits for another wave.

// A job as the narrow stream sees it, built once per call for every job of
// this CU (see build_jobs).  Lanes add their row, K-block and column.
struct JobDesc {
  uint64_t wb;        // weights of the job's row 0 (up/gate: gate row 8t; down: the expert's W_down)
  uint64_t sb;        // block scales of that row (FP8 up/gate: its 128-row block row; MXFP4: its row)
  uint32_t tile;      // up/gate: the tile of ti intermediates
  uint32_t jump;      // up/gate, ti = 8: rows between lane row 7 (gate) and lane row 8 (up), minus one;
                      // ti = 16: rows from a gate row to its up row
  uint32_t shi;       // FP8 up/gate: scale bytes from the gate rows' block row to the up rows'; MXFP4: scale bytes per row
  int32_t nkb;        // K-blocks
  int32_t fmt;        // 0 FP8, 1 MXFP4
  int32_t ncols;      // the group's columns
  int32_t cbase;      // its first column in the column table
  int32_t srow;       // MXFP4: the expert row of lane row 0 in the tiled scale bytes (up/gate: the tile's first gate row)
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
  d.srow = uni((int)c[3]);
  return d;
}

// The descriptor of an up/gate job (tile `tile` of the expert's ti-row gate
// and up tiles) or of a down job (the expert's whole W_down).
__device__ inline JobDesc make_desc(const Params& p, bool up, bool sh, int e, int tile, int ncols, int cbase) {
  const size_t H = p.H, I = p.I;
  JobDesc d;
  const int iexp = sh ? p.Is : p.I;
  const int kdim = up ? p.H : iexp;
  e -= p.ef;  // index into the routed weights held here
  d.fmt = sh ? 0 : p.routed_fmt;
  d.nkb = kdim / (d.fmt ? 256 : 128);  // K-blocks: 128 bytes of every row (128 FP8 or 256 MXFP4 values)
  d.ncols = ncols;
  d.cbase = cbase;
  d.srow = 0;
  const int lti = p.lti;
  d.jump = up ? (lti == 3 ? iexp - 8 : iexp) : 0;
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
      const int nb_lo = (tile << lti) / 128, nb_hi = (iexp + (tile << lti)) / 128;
      w += (size_t)(tile << lti) * kdim;
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
      w += (size_t)(tile << lti) * (kdim / 2);
      d.srow = tile << lti;  // the scales are addressed by expert row (tiled layout)
    }
  }
  d.wb = (uint64_t)w;
  d.sb = (uint64_t)S;
  return d;
}

// Up/gate (group, tile) pair j of the step: the shared tiles,
// then rt_tiles tiles per routed group.  Sets its group and tile.  A routed
// group's tiles are rotated by 37 per group, so that a CU's pairs fall on
// different row blocks of successive experts (unrotated, CU c reads row
// block c of every expert, and the phase ends were spread by XCD, up to
// 18 us apart at 64 rows; rotated: 64 rows 1379 -> 1348 us, 8 rows 234 ->
// 232 us, same-box A/B).  Any rotation keeps the tiles a permutation.
__device__ __forceinline__ void up_pair(const Params& p, const Sched& s, int j, int& g, int& tile) {
  if (j < s.sh_tiles) {
    g = 0;
    tile = j;
  } else {
    g = p.n_shared + (j - s.sh_tiles) / s.rt_tiles;
    tile = ((j - s.sh_tiles) % s.rt_tiles + (g - p.n_shared + 1) * 37) % s.rt_tiles;
  }
}

// Column tiles of a group of c columns: jobs of at most cpj columns each.
__device__ __forceinline__ int n_ctiles(const Params& p, int c) { return (c + p.cpj - 1) / p.cpj; }

// Up/gate jobs of a call: CU c takes the (group, tile) pairs c + q*ncu in
// order, and a pair is one job per column tile of its group (its weight rows
// are streamed once per column tile, back to back, the repeats mostly from
// the caches).  Inside the CU a job is cut into chunks, one per K-phase w
// (K-blocks w + 8i), and the waves claim chunks in order from an LDS
// counter.  A chunk's partial is the same sum whichever wave forms it, so
// the job's sum over its K-phases in order does not depend on which wave did
// what, and waves that stream faster take more chunks.

// This CU's shared-expert pairs (dealt c, c + ncu, ...) and their jobs.
__device__ __forceinline__ int shared_pairs_here(const Params& p) {
  const int sh_tiles = p.n_shared ? p.Is >> p.lti : 0;
  return (int)blockIdx.x < sh_tiles ? (sh_tiles - 1 - (int)blockIdx.x) / p.ncu + 1 : 0;
}
__device__ __forceinline__ int shared_jobs_here(const Params& p) { return shared_pairs_here(p) * n_ctiles(p, p.T); }

// The stream's state and the tables of this CU's shared-expert jobs (local
// jobs 0..nS-1; they need no routing).  Whole workgroup, plain per-thread
// LDS accesses; the caller synchronises.
__device__ inline void stream_init(const Params& p, const Lds& L, int nS) {
  const int tid = threadIdx.x;
  const int nct = n_ctiles(p, p.T);
  for (int k = tid; k < nS; k += kThreads) {
    const int q = k / nct, ct = k - q * nct;
    const int nc = p.T - ct * p.cpj < p.cpj ? p.T - ct * p.cpj : p.cpj;
    L.jd[k] = make_desc(p, true, true, 0, (int)blockIdx.x + q * p.ncu, nc, ct * p.cpj);
  }
  if (p.n_shared && tid < p.T) {
    L.cols[tid] = tid * 16 + p.K;
    L.cgrp[tid] = 0;
  }
  if (tid < kPuWin) {
    L.wcnt[tid] = 0u;
    L.wgen[tid] = 0u;
  }
  if (tid == 0) {
    L.ccnt[0] = 0u;
    L.ccnt[1] = 0u;
    L.misc[kMiscReady] = 0;
    L.misc[kMiscRouted] = 0;
    L.misc[kMiscPolled] = 0;
  }
}

// Exclusive offsets of per-lane counts n over the wave, added to `base`
// (which moves on by the wave's total).
__device__ __forceinline__ int wave_offset(int n, int& base) {
  const int v = wave_incl_scan(n);
  const int o = base + v - n;
  base += __builtin_amdgcn_readlane(v, 63);
  return o;
}

// The tables that need the routing, written by one wave:
//   PART 1: the routed up/gate jobs (local jobs nS.., this CU's routed pairs
//           in order, each pair's column tiles in order), then nU;
//   PART 2: the down jobs at qcap + i (each group's column tiles, groups in
//           order), then nD.
template <int PART>
__device__ inline void routed_tables(const Params& p, const Lds& L, const Sched& s, int nS) {
  const int lane = threadIdx.x & 63;
  if (PART & 1) {
    // this CU's first routed pair: the smallest j >= sh_tiles with
    // j = blockIdx.x (mod ncu)
    const int r = s.sh_tiles % p.ncu;
    const int first = s.sh_tiles + (((int)blockIdx.x - r) % p.ncu + p.ncu) % p.ncu;
    int base = nS;
    for (int j0 = first; j0 < s.n_pairs; j0 += 64 * p.ncu) {
      const int j = j0 + lane * p.ncu;
      int g = 0, tile = 0, c = 0, nct = 0;
      if (j < s.n_pairs) {
        up_pair(p, s, j, g, tile);
        c = L.gcnt[g];
        nct = n_ctiles(p, c);
      }
      const int off = wave_offset(nct, base);
      for (int ct = 0; ct < nct; ++ct) {
        const int nc = c - ct * p.cpj < p.cpj ? c - ct * p.cpj : p.cpj;
        L.jd[off + ct] = make_desc(p, true, false, L.gexp[g], tile, nc, L.gstart[g] + ct * p.cpj);
      }
    }
    if (lane == 0) L.misc[kMiscNU] = base;
  }
  if (PART & 2) {
    int base = 0;
    for (int g0 = 0; g0 < s.G; g0 += 64) {
      const int g = g0 + lane;
      const bool sh = shared_group(p, g);
      const int c = g < s.G ? (sh ? p.T : L.gcnt[g]) : 0;
      const int nct = n_ctiles(p, c);
      const int off = wave_offset(nct, base);
      for (int ct = 0; ct < nct; ++ct) {
        const int nc = c - ct * p.cpj < p.cpj ? c - ct * p.cpj : p.cpj;
        L.jd[p.qcap + off + ct] =
            make_desc(p, false, sh, sh ? 0 : L.gexp[g], 0, nc, (sh ? 0 : L.gstart[g]) + ct * p.cpj);
      }
    }
    if (lane == 0) L.misc[kMiscND] = base;
  }
}

// Per-wave constants of a phase (KIND 1 up/gate, 2 down split by K-phase,
// 3 down by claimed whole jobs).  Up/gate: every wave takes K-blocks w + 8i
// of each job; in a one-tile item rows 0..7 are gate rows and 8..15 up rows,
// in a two-tile item tile A holds 16 gate rows and tile B their up rows.
// Down (KIND 2): wave w takes tile rt of the CU's slice, rows hb.. (nlive
// live), and with two-tile items tile rt + 1 too (hb2, nlive2), and its
// K-phase's K-blocks (see ksplit_phase).  KIND 3: a claimed unit's tiles and
// all its K-blocks (the constants are set per unit).
struct PhaseN {
  int k0, lstep;  // this wave's K-blocks: k0 + (i << lstep)
  int hb, nlive;  // down: first row of this wave's tile and its live rows
  int split;      // FP8: MFMA output rows (4*lg + q) below it take the first scale block row
  int dnb;        // FP8 down: block rows between the tile's first and last live row (0 or 1)
  int rt;         // down: this wave's tile
  int hb2, nlive2, split2, dnb2;  // two-tile K-split down: tile B (tile rt + 1); nlive2 <= 0: none
  int nw;         // up/gate: waves with items (min(K-blocks, 8))
  int nsc, nct;   // up/gate: chunks of the CU's shared-expert jobs, column tiles per shared pair
  int js, jp;     // K-split down: the wave takes the down jobs j with j mod js == jp
  int h0, hc, nrt;  // KIND 3: this CU's slice and its 16-row tiles
};
template <int KIND>
__device__ __forceinline__ int ph_k0(const PhaseN& ph) { return KIND == 1 ? wave_id() : ph.k0; }
template <int KIND>
__device__ __forceinline__ int ph_lstep(const PhaseN& ph) { return KIND == 1 ? 3 : ph.lstep; }
template <int KIND, int WT>
__device__ __forceinline__ int ph_split(const PhaseN& ph) { return KIND == 1 ? (WT == 2 ? 16 : 8) : ph.split; }
// a two-tile item's tile B: up/gate, all up rows (the second scale word of
// s2, which repeats s); down, its own rows
template <int KIND>
__device__ __forceinline__ int ph_split2(const PhaseN& ph) { return KIND == 1 ? 0 : ph.split2; }

// The down constants of tile rt of the slice [h0, h0 + hc), K-blocks
// k0 + (i << lstep).
__device__ __forceinline__ PhaseN down_phase(int h0, int hc, int nrt, int rt, int k0, int lstep) {
  PhaseN ph;
  ph.rt = rt;
  ph.k0 = k0;
  ph.lstep = lstep;
  ph.hb = h0 + 16 * rt;
  ph.nlive = hc - 16 * rt < 16 ? hc - 16 * rt : 16;
  ph.split = (ph.hb / 128 + 1) * 128 - ph.hb;  // a 16-row tile spans at most two scale block rows
  ph.dnb = ph.nlive > 0 ? ((ph.hb + ph.nlive - 1) >> 7) - (ph.hb >> 7) : 0;
  ph.hb2 = ph.hb + 16;
  ph.nlive2 = 0;
  ph.split2 = 0;
  ph.dnb2 = 0;
  ph.nw = 0;
  ph.js = 1;
  ph.jp = 0;
  ph.h0 = h0;
  ph.hc = hc;
  ph.nrt = nrt;
  return ph;
}

// Down constants of the unit of 16-row tiles 2*pr and 2*pr + 1 of the slice
// (tile B empty past the slice's tiles).
__device__ __forceinline__ PhaseN down_pair(int h0, int hc, int nrt, int pr, int k0, int lstep) {
  PhaseN ph = down_phase(h0, hc, nrt, 2 * pr, k0, lstep);
  const PhaseN b = down_phase(h0, hc, nrt, 2 * pr + 1, 0, 0);
  ph.hb2 = b.hb;
  ph.nlive2 = b.nlive;
  ph.split2 = b.split;
  ph.dnb2 = b.dnb;
  return ph;
}

// The K-split down constants of wave w: tile w mod nrt_p of the CU's slice
// and K-phase (w / nrt_p) of the kph phases.  When a down job has fewer
// K-blocks than kph (a small intermediate size), the phases are cut to the
// power of two kpe >= the most K-blocks a down job has, and the waves left
// over take every (kph/kpe)-th job instead, so no wave idles.  Each phase
// then holds at most one K-block, as it did with kph phases: the partials,
// and their phase-order sum, are the same bits.
//
// WT = 2 (two-tile items): a wave takes tiles 2i and 2i+1 together (pair i =
// w mod nrt_p/2) on one activation operand, and the two waves that would
// have taken them in the same K-phase take alternate jobs instead.  Each
// (tile, K-phase) partial is the same chain over the same K-blocks, so the
// products keep their bits.  With one tile (nrt_p = 1) tile B is empty.
template <int WT>
__device__ __forceinline__ PhaseN ksplit_phase(const Params& p, const Sched& s, int w) {
  const int nkb_rt = p.I / (p.routed_fmt ? 256 : 128), nkb_sh = p.n_shared ? p.Is / 128 : 0;
  const int nkb = nkb_rt > nkb_sh ? nkb_rt : nkb_sh;
  int kpe = 1;
  while (kpe < nkb && kpe < s.kph) kpe <<= 1;
  if (WT == 1 || s.nrt_p == 1) {
    const int q = w / s.nrt_p;
    PhaseN ph = down_phase(s.h0, s.hc, s.nrt, w % s.nrt_p, q % kpe, 31 - __builtin_clz(kpe));
    ph.js = s.kph / kpe;
    ph.jp = q / kpe;
    return ph;
  }
  const int npair = s.nrt_p >> 1, rest = w / npair, q = rest % s.kph;
  PhaseN ph = down_phase(s.h0, s.hc, s.nrt, 2 * (w % npair), q % kpe, 31 - __builtin_clz(kpe));
  const PhaseN b = down_phase(s.h0, s.hc, s.nrt, 2 * (w % npair) + 1, 0, 0);
  ph.hb2 = b.hb;
  ph.nlive2 = b.nlive;
  ph.split2 = b.split;
  ph.dnb2 = b.dnb;
  ph.js = 2 * (s.kph / kpe);
  ph.jp = q / kpe + (s.kph / kpe) * (rest / s.kph);
  return ph;
}


template <int KIND>
__device__ __forceinline__ int job_items(const PhaseN& ph, int nkb) {
  const int k0 = ph_k0<KIND>(ph);
  return nkb > k0 ? ((nkb - 1 - k0) >> ph_lstep<KIND>(ph)) + 1 : 0;
}

// The fetch side: byte offsets of this lane's next item from uniform bases.
struct FetchN {
  int k;                         // next job to set up (down); KIND 3: the claimed unit, -1 before the first
  int kp, nkb;                   // KIND 3: the unit's K-phase being fetched, and its K-blocks
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
  uint32_t h2;                   // MXFP4 items: the second half's activation offset (FP8 items: 0)
  uint32_t wj, sj;               // two-tile items: bytes from a tile-A row's weights (MXFP4: scales) to its tile-B row's
};

// Weight tiles per item (see stream_ti): up/gate items of a kernel with
// MXFP4 routed experts and two activation loads are two 16-row tiles (gate
// rows, then their up rows) on one activation operand; every other item is
// one tile.
// Down items are two 16-row down tiles of the CU's slice on one activation
// operand (see ksplit_phase and fetch_next_dc).
// W2: the up/gate items of an FP8 kernel are two tiles too (above
// kKsplitRows rows, see stream_ti).
template <int FMT, int KIND, int AL, bool W2 = false>
constexpr int item_wt() { return (AL == 2 && (FMT != 0 || W2) && KIND == 1) || KIND != 1 ? 2 : 1; }

// One item: a K-block of a 16-row tile, 128 bytes of each row (FP8: 128
// values, one fp32 block scale per 128-row block; MXFP4: 256 values, the
// lane's two E8M0 scales in s).  B: the activations, AL loads per 128
// values (2*AL in a kernel with MXFP4 experts, whose FP8 items repeat the
// first AL as the second).
struct ItemN {
  u32x4 w0, w1, w2, w3, B[8];  // w2, w3: a two-tile item's tile B
  uint32_t s, s2;
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

// Byte offset of expert row n's K-block kb in tiled MXFP4 scale bytes (16
// rows of one K-block are one 128-byte line; nkb K-blocks per row).
__device__ __forceinline__ uint32_t mx_soff(uint32_t n, uint32_t nkb, uint32_t kb) {
  return ((lmul(n >> 4, nkb) + kb) << 7) + ((n & 15u) << 3);
}

// Sets the fetch side to job descriptor d, whose first item is this wave's
// K-block k0; `code` is this lane's column (row*16 + slot), n its items.
template <int FMT, int KIND, int AL, bool W2 = false>
__device__ __forceinline__ void fetch_from_desc(const Params& p, const PhaseN& ph, FetchN& f, const JobDesc& d, int k0,
                                                int n, int code) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const int fmt = FMT == 0 ? 0 : d.fmt;
  constexpr int WT = item_wt<FMT, KIND, AL, W2>();
  const uint32_t lrow = KIND == 1 ? (WT == 2 ? row : row < 8 ? row : row + d.jump)
                                  : ph.hb + (row < ph.nlive ? row : ph.nlive - 1);
  // down tile B's rows (its last live row repeated, or tile A's rows if
  // it has none)
  const uint32_t lrow2 = WT == 2 && KIND != 1 && ph.nlive2 > 0
                             ? (uint32_t)(ph.hb2 + (row < ph.nlive2 ? row : ph.nlive2 - 1))
                             : lrow;
  // A kernel with MXFP4 experts loads a two-tile item's scales with one
  // load (s): see eat_item_n.
  constexpr bool M2 = FMT != 0 && WT == 2;
  f.wb = (const uint8_t*)d.wb;
  // 128 bytes of each row per K-block, 32 per lane group
  f.wo = lmul(lrow, (uint32_t)(d.nkb * 128)) + (uint32_t)k0 * 128u + (uint32_t)lg * 32u;
  if (fmt == 0) {
    if (KIND == 1) {
      f.sb = (const uint8_t*)d.sb;
      f.so = (lane < 32 ? 0u : d.shi) + 4u * (uint32_t)k0;
    } else if (M2) {
      // one block-scale word per lane quarter: tile A's first and second
      // block row, then tile B's (tile A's again if tile B has no rows)
      f.sb = (const uint8_t*)d.sb + 4 * (size_t)(ph.hb >> 7) * d.nkb;
      const uint32_t b2 = ph.nlive2 > 0 ? 4u * (uint32_t)(((ph.hb2 >> 7) - (ph.hb >> 7)) * d.nkb) : 0u;
      const uint32_t d2 = 4u * (uint32_t)((ph.nlive2 > 0 ? ph.dnb2 : ph.dnb) * d.nkb);
      f.so = (lg == 0 ? 0u : lg == 1 ? 4u * (uint32_t)(ph.dnb * d.nkb) : lg == 2 ? b2 : b2 + d2) + 4u * (uint32_t)k0;
    } else {
      f.sb = (const uint8_t*)d.sb + 4 * (size_t)(ph.hb >> 7) * d.nkb;
      f.so = (lane < 32 ? 0u : 4u * (uint32_t)(ph.dnb * d.nkb)) + 4u * (uint32_t)k0;
    }
  } else if (M2) {
    // lane groups 0 and 1 take words 0 and 1 (bytes 0..7) of tile A's row,
    // groups 2 and 3 those of tile B's row
    f.sb = (const uint8_t*)d.sb;
    const uint32_t na = (uint32_t)d.srow + lrow, nb = KIND == 1 ? na + d.jump : lrow2;
    f.so = mx_soff(lg < 2 ? na : nb, (uint32_t)d.nkb, (uint32_t)k0) + 4u * (uint32_t)(lg & 1);
  } else {
    // the K-block's 8 scale bytes of the row: lane group lg takes bytes
    // 2lg and 2lg+1, from the aligned word 4*(lg >> 1)
    f.sb = (const uint8_t*)d.sb;
    f.so = mx_soff((uint32_t)d.srow + lrow, (uint32_t)d.nkb, (uint32_t)k0) + 4u * (uint32_t)(lg >> 1);
  }
  // a lane's first piece: j = lane mod G; an MXFP4 K-block is 256 values,
  // 64 per lane group
  f.ao = 2 * act_offset(p, KIND, code, lg) + (fmt ? 64u * (uint32_t)lg : 0u) + (fmt ? 512u : 256u) * (uint32_t)k0 +
         16u * (uint32_t)(lane & (4 / AL - 1));
  f.h2 = fmt ? 64u : 0u;
  f.fmt = fmt;
  f.nstep = 1 << ph_lstep<KIND>(ph);
  f.left = n;
  if (WT == 2 && KIND == 1) {
    f.wj = d.jump * (uint32_t)(d.nkb * 128);
    f.sj = 0u;  // (an FP8 kernel's up/gate s2 repeats s)
  } else if (WT == 2) {
    // tile B's weights from tile A's: not negative
    f.wj = lmul(lrow2 - lrow, (uint32_t)(d.nkb * 128));
    if (M2) {
      f.sj = 0u;
    } else if (fmt == 0) {
      const uint32_t so2 = ph.nlive2 > 0 ? 4u * (uint32_t)(((ph.hb2 >> 7) - (ph.hb >> 7)) * d.nkb) +
                                               (lane < 32 ? 0u : 4u * (uint32_t)(ph.dnb2 * d.nkb)) + 4u * (uint32_t)k0
                                         : f.so;
      f.sj = so2 - f.so;
    } else {
      f.sj = mx_soff(lrow2, (uint32_t)d.nkb, 0u) - mx_soff(lrow, (uint32_t)d.nkb, 0u);
    }
  } else {
    f.wj = 0u;
    f.sj = 0u;
  }
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
  f.h2 = 0;
  f.fmt = 0;
  f.nstep = 0;
  f.left = 1 << 30;
  f.wj = 0;
  f.sj = 0;
}

// Down: moves the fetch side to the next job of [f.k, kend) with items for
// this wave, or past the end.
template <int FMT, int KIND, int AL>
__device__ inline void fetch_next_n(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int kend) {
  for (; f.k < kend; ++f.k) {
    if (KIND == 2 && ((f.k - p.qcap) & (ph.js - 1)) != ph.jp) continue;
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
// Chunk c's job and K-phase.  The column-tile jobs of one shared-expert pair
// (the same weight rows for different columns) are taken phase by phase,
// all tiles' phase 0, then phase 1, ..., so a K-block's repeats follow each
// other closely and come from the caches; every other job's chunks are
// taken job by job.
__device__ __forceinline__ void chunk_map(uint32_t c, const PhaseN& ph, int& q, int& kp) {
  if ((int)c < ph.nsc && ph.nct > 1) {
    const int per = ph.nct * ph.nw;
    const int pi = (int)c / per, i = (int)c - pi * per;
    kp = i / ph.nct;
    q = pi * ph.nct + (i - kp * ph.nct);
  } else {
    q = chunk_job(c, ph.nw);
    kp = (int)c - q * ph.nw;
  }
}
template <int FMT, int AL, bool W2 = false>
__device__ inline void fetch_next_up(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int nS, bool& ok) {
  const uint32_t c = lds_inc_lane0(L.ccnt);
  int q, kp;
  chunk_map(c, ph, q, kp);
  if (q >= nS && f.nu < 0) {
    lds_wait<1>(p, (const uint32_t*)L.misc + kMiscReady, 1u, ok);
    f.nu = ok ? lds_ldi_uniform(L.misc + kMiscNU) : 0;
  }
  if (q < (q < nS ? nS : f.nu)) {
    const JobDesc d = read_desc(L, q);
    lds_st32(L.cfifo + wave_id() * 8 + (f.nch & 7), c);
    f.nch = f.nch + 1;
    fetch_from_desc<FMT, 1, AL, W2>(p, ph, f, d, kp, ((d.nkb - 1 - kp) >> 3) + 1, lane_code<AL>(L, d));
    return;
  }
  fetch_dead(p, f);
}

// Items of K-phase kp of a down job of nkb K-blocks split into 1 << lkph
// phases (K-blocks kp + (i << lkph)).
__device__ __forceinline__ int phase_items(int nkb, int kp, int lkph) {
  return nkb > kp ? ((nkb - 1 - kp) >> lkph) + 1 : 0;
}

// Claimed down (KIND 3): moves the fetch side to the next K-phase with
// items of the wave's unit, or claims this CU's next down unit u (down entry
// u / npu, tiles 2*pr and 2*pr + 1 of the slice for pr = u mod npu, npu =
// the slice's pairs of 16-row tiles) and hands u on to the
// multiplying side; past the end once u reaches nunits.  A unit's K-blocks
// are fetched phase by phase (kp + kph*i for kp = 0, 1, ..), the order in
// which its sum is formed (see dc_phase_end).
template <int FMT, int AL>
__device__ inline void fetch_next_dc(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int nunits) {
  const int kph = 1 << ph.lstep;
  for (;;) {
    if (f.k >= 0) {
      for (int kp = f.kp + 1; kp < kph; ++kp) {
        const int n = phase_items(f.nkb, kp, ph.lstep);
        if (n > 0) {
          f.kp = kp;
          const int npu = (ph.nrt + 1) >> 1, ent = f.k / npu, pr = f.k - ent * npu;
          const JobDesc d = read_desc(L, p.qcap + ent);
          const PhaseN q = down_pair(ph.h0, ph.hc, ph.nrt, pr, kp, ph.lstep);
          fetch_from_desc<FMT, 2, AL>(p, q, f, d, kp, n, lane_code<AL>(L, d));
          return;
        }
      }
    }
    const uint32_t u = lds_inc_lane0(L.ccnt + 1);
    if ((int)u >= nunits) {
      f.k = -1;
      fetch_dead(p, f);
      return;
    }
    lds_st32(L.cfifo + wave_id() * 8 + (f.nch & 7), u);
    f.nch = f.nch + 1;
    f.k = (int)u;
    f.kp = -1;
    f.nkb = read_desc(L, p.qcap + (int)u / ((ph.nrt + 1) >> 1)).nkb;
  }
}

// kend: up/gate, the CU's shared-expert job count; down (KIND 2), the end of
// its job range; KIND 3, its unit count.
template <int FMT, int KIND, int AL, bool W2 = false>
__device__ __forceinline__ void fetch_next_any(const Params& p, const Lds& L, const PhaseN& ph, FetchN& f, int kend,
                                               bool& ok) {
  if (KIND == 1) fetch_next_up<FMT, AL, W2>(p, L, ph, f, kend, ok);
  else if (KIND == 3) fetch_next_dc<FMT, AL>(p, L, ph, f, kend);
  else fetch_next_n<FMT, KIND, AL>(p, L, ph, f, kend);
}

template <int FMT, int WT>
__device__ __forceinline__ void fetch_weights_n(const FetchN& f, ItemN& it) {
  const uint8_t* w = f.wb + f.wo;
  it.w0 = ldg<u32x4>(w);
  it.w1 = ldg<u32x4>(w + 16);
  if (WT == 2) {
    it.w2 = ldg<u32x4>(w + f.wj);
    it.w3 = ldg<u32x4>(w + f.wj + 16);
  }
  it.s = ldg<uint32_t>(f.sb + f.so);
  // an FP8 kernel's tile B scales: a down tile B's block rows; an up/gate
  // item loads s again (the up rows' block scale is lane 32's word of s).
  // A kernel with MXFP4 experts has both tiles' scales in s.
  if (WT == 2 && FMT == 0) it.s2 = ldg<uint32_t>(f.sb + (uint32_t)(f.so + f.sj));
}
// Activations: AL loads of 16 B per lane per 128 values, pieces j + G*i
// (the load instructions, not the bytes, are what the vector memory path
// pays for).  A kernel with MXFP4 experts issues 2*AL: the second half at
// h2 (64 B on: pieces 4.. of the lane group's 8), or again the first half
// for an FP8 item (h2 = 0), so that every item issues the same loads.
template <int FMT, int AL>
__device__ __forceinline__ void fetch_acts_n(const uint8_t* ab, uint32_t ao, uint32_t h2, ItemN& it) {
  const uint8_t* a = ab + ao;
#pragma unroll
  for (int i = 0; i < AL; ++i) it.B[i] = ldg<u32x4>(a + 16 * (4 / AL) * i);
  if (FMT != 0) {
#pragma unroll
    for (int i = 0; i < AL; ++i) it.B[AL + i] = ldg<u32x4>(a + h2 + 16 * (4 / AL) * i);
  }
}
template <int FMT, int AL, int WT>
__device__ __forceinline__ void fetch_item_n(const FetchN& f, ItemN& it) {
  fetch_weights_n<FMT, WT>(f, it);
  fetch_acts_n<FMT, AL>(f.ab, f.ao, f.h2, it);
}

template <int FMT>
__device__ __forceinline__ void fetch_adv_n(FetchN& f) {
  const uint32_t n = (uint32_t)uni(f.nstep);
  const bool mx = FMT != 0 && f.fmt != 0;
  f.wo += n * 128u;
  f.so += (mx ? 128u : 4u) * n;
  f.ao += (mx ? 512u : 256u) * n;
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
  int split;       // KIND 3: the job's FP8 scale split (see PhaseN)
  int split2;      // KIND 3: the same for the unit's tile B
  bool pst2;       // KIND 3: the unit has a tile B
  int kp, nkb;     // KIND 3: the K-phase being multiplied, and the unit's K-blocks
};

// Down: moves the multiplying side to its next job of [e.k, kend) with
// items; false at the end.
template <int FMT, int KIND, int AL>
__device__ inline bool eat_next_n(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, int kend) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane_col<AL>(lane);
  for (; e.k < kend; ++e.k) {
    if (KIND == 2 && ((e.k - p.qcap) & (ph.js - 1)) != ph.jp) continue;
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
template <int FMT, int AL, bool W2 = false>
__device__ inline bool eat_next_up(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, int fnch) {
  if (e.nch >= fnch) return false;
  const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane_col<AL>(lane);
  const uint32_t c = (uint32_t)lds_ldi_uniform((const int32_t*)L.cfifo + wave_id() * 8 + (e.nch & 7));
  e.nch = e.nch + 1;
  int q, kp;
  chunk_map(c, ph, q, kp);
  const JobDesc d = read_desc(L, q);
  e.q = q;
  e.left = ((d.nkb - 1 - kp) >> 3) + 1;
  e.fmt = FMT == 0 ? 0 : d.fmt;
  e.pst = col < d.ncols && (lane & (4 / AL - 1)) == 0;
  e.pidx = ((((uint32_t)q & (kPuWin - 1)) * kWaves + (uint32_t)kp) * (uint32_t)p.pcols + (uint32_t)col) *
               (16u * (uint32_t)item_wt<FMT, 1, AL, W2>()) +
           4u * (uint32_t)lg;
  return true;
}

// Claimed down (KIND 3): moves the multiplying side to the next unit the
// fetch side has claimed, at its first K-phase; false at the end.  The
// unit's sums go to Pd[0][row][slot] at its two tiles.
template <int FMT, int AL>
__device__ inline bool eat_next_dc(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, int fnch) {
  if (e.nch >= fnch) return false;
  const int lane = threadIdx.x & 63, lg = lane >> 4, col = lane_col<AL>(lane);
  const uint32_t u = (uint32_t)lds_ldi_uniform((const int32_t*)L.cfifo + wave_id() * 8 + (e.nch & 7));
  e.nch = e.nch + 1;
  const int npu = (ph.nrt + 1) >> 1, ent = (int)u / npu, pr = (int)u - ent * npu;
  const JobDesc d = read_desc(L, p.qcap + ent);
  const PhaseN q = down_pair(ph.h0, ph.hc, ph.nrt, pr, 0, 0);
  e.nkb = d.nkb;
  e.kp = 0;
  e.left = phase_items(d.nkb, 0, ph.lstep);
  e.fmt = FMT == 0 ? 0 : d.fmt;
  e.pst = col < d.ncols && (lane & (4 / AL - 1)) == 0;
  const int code = lane_code<AL>(L, d);
  e.pidx = lmul(lmul((uint32_t)(code >> 4), (uint32_t)(p.K + 1)) + (uint32_t)(code & 15), (uint32_t)p.pitch) +
           32u * (uint32_t)pr + 4u * (uint32_t)lg;
  e.split = q.split;
  e.split2 = q.split2;
  e.pst2 = e.pst && q.nlive2 > 0;
  return true;
}

// Claimed down: the end of a K-phase's items.  The phase's partial (an FMA
// chain over its K-blocks, as one wave forms it when the phases are split
// over waves) is added to the unit's sum, which starts at +0 and takes the
// phases in order, a phase without items adding +0: the sum a split down
// job's products get in the combine.  Moves to the next phase with items,
// or at the unit's end stores the sum (unit_end) and starts the next unit;
// false once no unit is left.
// Both tiles of the unit (tile B: acc2, tot2) alike.
template <int FMT, int AL>
__device__ inline bool dc_phase_end(const Params& p, const Lds& L, const PhaseN& ph, EatN& e, f32x4& acc, f32x4& tot,
                                    f32x4& acc2, f32x4& tot2, int fnch, bool& unit_end) {
  const int kph = 1 << ph.lstep;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    tot[q] += acc[q];
    tot2[q] += acc2[q];
  }
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
  unit_end = false;
  for (int kp = e.kp + 1; kp < kph; ++kp) {
    const int n = phase_items(e.nkb, kp, ph.lstep);
    if (n > 0) {
      e.kp = kp;
      e.left = n;
      return true;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tot[q] += 0.f;
      tot2[q] += 0.f;
    }
  }
  unit_end = true;
  if (e.pst) lds_st128(L.pbuf + e.pidx, __builtin_bit_cast(u32x4, tot));
  if (e.pst2) lds_st128(L.pbuf + e.pidx + 16, __builtin_bit_cast(u32x4, tot2));
  tot = f32x4{0.f, 0.f, 0.f, 0.f};
  tot2 = f32x4{0.f, 0.f, 0.f, 0.f};
  return eat_next_dc<FMT, AL>(p, L, ph, e, fnch);
}

// Up/gate job q is complete in partial window win (waves 0..nw-1 stored):
// every (column, intermediate) is summed over the 8 waves in order (a wave
// without items adds zero), gate and up, and its SwiGLU value goes to mid as
// bf16.  One wave; lane = (column, pair of intermediates); a column's 8*WT
// gate rows come first, then their up rows.
template <int WT>
__device__ inline void up_reduce_job(const Params& p, const Lds& L, int q, int win, int nw) {
  const JobDesc d = read_desc(L, q);
  constexpr int per = 4 * WT;  // pairs of intermediates per column
  const int lane = threadIdx.x & 63, col = lane / per, i2 = 2 * (lane % per);
  if (col < d.ncols) {
    const size_t wstride = (size_t)p.pcols * 16 * WT;
    const float* pu = L.pbuf + ((size_t)win * kWaves * p.pcols + col) * 16 * WT + i2;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f32x2 gv = {0.f, 0.f}, uv = {0.f, 0.f};
      if (w < nw) {
        gv = lds_get<f32x2>(pu + w * wstride);
        uv = lds_get<f32x2>(pu + w * wstride + 8 * WT);
      }
      g0 += gv[0];
      g1 += gv[1];
      u0 += uv[0];
      u1 += uv[1];
    }
    const float m0 = swiglu(g0, u0), m1 = swiglu(g1, u1);
    if (!isfinite(m0) || !isfinite(m1)) set_err(p.err, kErrMid);
    const int code = lds_get<int32_t>(L.cols + d.cbase + col);
    st_agent<uint32_t>(p.mid + ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.mid_ld + 8 * WT * d.tile + i2,
                       f32_to_bf16_rne(m0) | (f32_to_bf16_rne(m1) << 16));
  }
}

// The end of a chunk of up/gate job e.q: once the window's previous job is
// summed, store the chunk's partial tile and arrive; the wave that ends the
// job's last (nw-th) chunk sums the job and frees the window.
template <int WT>
__device__ inline void up_job_end(const Params& p, const Lds& L, const EatN& e, const f32x4& acc, const f32x4& acc2,
                                  int nw, bool& ok) {
  const int win = e.q & (kPuWin - 1);
  lds_wait<1>(p, L.wgen + win, (uint32_t)(e.q / kPuWin), ok);
  if (e.pst) {
    lds_st128(L.pbuf + e.pidx, __builtin_bit_cast(u32x4, acc));
    if (WT == 2) lds_st128(L.pbuf + e.pidx + 16, __builtin_bit_cast(u32x4, acc2));
  }
  if (lds_inc_lane0(L.wcnt + win) == (uint32_t)nw - 1) {
    up_reduce_job<WT>(p, L, e.q, win, nw);
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
      switch (m & 3) {
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

// split / split2: MFMA output rows (4*lg + q) of tile A / tile B below it
// take lane 0's scale word of s / s2, the others lane 32's (FP8).
// Q4 (two-tile items in a kernel with MXFP4 experts): an FP8 item holds
// tile A's two block-scale words at lanes 0 and 16 of s and tile B's at
// lanes 32 and 48; an MXFP4 item holds words 0 and 1 of each row's scale
// bytes for tile A in lane groups 0 and 1 and for tile B in groups 2 and 3,
// which two row-swap steps hand to the lanes that use them.
template <int F, int AL, int WT, bool Q4 = false>
__device__ __forceinline__ void eat_item_n(int split, int split2, int lg, const ItemN& it, f32x4& acc, f32x4& acc2) {
  bf16x8 A[4];
  if (F == 0 && WT == 1) {
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
  } else if (F == 0) {
    // two tiles on one activation operand: up/gate, tile A the gate rows
    // (lane 0's word of s) and tile B their up rows (lane 32's word of s2 =
    // s); down, two 16-row tiles with scale words of their own
    bf16x8 Bm[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) Bm[m] = act_operand<AL>(it, m);
    const float s_lo = __int_as_float(__builtin_amdgcn_readlane((int)it.s, 0));
    const float s_hi = __int_as_float(__builtin_amdgcn_readlane((int)it.s, Q4 ? 16 : 32));
    const float s2_lo = __int_as_float(__builtin_amdgcn_readlane((int)(Q4 ? it.s : it.s2), Q4 ? 32 : 0));
    const float s2_hi = __int_as_float(__builtin_amdgcn_readlane((int)(Q4 ? it.s : it.s2), Q4 ? 48 : 32));
    A[0] = e4m3x8_to_bf16(it.w0[0], it.w0[1]);
    A[1] = e4m3x8_to_bf16(it.w0[2], it.w0[3]);
    A[2] = e4m3x8_to_bf16(it.w1[0], it.w1[1]);
    A[3] = e4m3x8_to_bf16(it.w1[2], it.w1[3]);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) t = mfma16(A[m], Bm[m], t);
    A[0] = e4m3x8_to_bf16(it.w2[0], it.w2[1]);
    A[1] = e4m3x8_to_bf16(it.w2[2], it.w2[3]);
    A[2] = e4m3x8_to_bf16(it.w3[0], it.w3[1]);
    A[3] = e4m3x8_to_bf16(it.w3[2], it.w3[3]);
    f32x4 t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) t2 = mfma16(A[m], Bm[m], t2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q] = fmaf(t[q], 4 * lg + q < split ? s_lo : s_hi, acc[q]);
      acc2[q] = fmaf(t2[q], 4 * lg + q < split2 ? s2_lo : s2_hi, acc2[q]);
    }
  } else if (WT == 1) {
    // 256 values: lane group lg holds values 64lg.. (w0: the first 32 with
    // scale byte 2lg, w1: the next 32 with byte 2lg+1); MFMA m takes
    // values 64lg + 8m.. of every lane group
    const uint32_t sh = 16u * (uint32_t)(lg & 1);
    const float sc0 = e8m0_to_f32((it.s >> sh) & 0xffu), sc1 = e8m0_to_f32((it.s >> (sh + 8)) & 0xffu);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w0[m], sc0);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = mfma16(A[m], act_operand<AL>(it, m), acc);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w1[m], sc1);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = mfma16(A[m], act_operand<AL>(it, 4 + m), acc);
  } else {
    // the same for two tiles (tile B with its own scale bytes s2)
    bf16x8 Bm[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) Bm[m] = act_operand<AL>(it, m);
    const uint32_t sh = 16u * (uint32_t)(lg & 1);
    // lane group g gets word g >> 1 of its row's bytes for each tile
    // (row r of lane group g: lane 16g + r)
    const auto x = __builtin_amdgcn_permlane32_swap(it.s, it.s, false, false);  // groups (0,1,0,1), (2,3,2,3)
    const auto ta = __builtin_amdgcn_permlane16_swap(x[0], x[0], false, false);  // all groups 0, all 1
    const auto tb = __builtin_amdgcn_permlane16_swap(x[1], x[1], false, false);  // all groups 2, all 3
    const uint32_t sa = lg < 2 ? ta[0] : ta[1], sb = lg < 2 ? tb[0] : tb[1];
    {
      const float sc0 = e8m0_to_f32((sa >> sh) & 0xffu), sc1 = e8m0_to_f32((sa >> (sh + 8)) & 0xffu);
#pragma unroll
      for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w0[m], sc0);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma16(A[m], Bm[m], acc);
#pragma unroll
      for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w1[m], sc1);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma16(A[m], Bm[4 + m], acc);
    }
    {
      const float sc0 = e8m0_to_f32((sb >> sh) & 0xffu), sc1 = e8m0_to_f32((sb >> (sh + 8)) & 0xffu);
#pragma unroll
      for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w2[m], sc0);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc2 = mfma16(A[m], Bm[m], acc2);
#pragma unroll
      for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(it.w3[m], sc1);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc2 = mfma16(A[m], Bm[4 + m], acc2);
    }
  }
}

// One phase of the narrow stream over jobs [k, kend) of the job tables, in
// pieces: ring_open sets the fetch side to the first job, ring_fill issues
// the first D items (all loads, or weights and scales only, the
// activations following in ring_fill_acts), and ring_run multiplies and
// refills until the last job has ended.  Partials go to LDS, which must be
// zero where this wave has no items.
constexpr int kRingD = 5;   // up/gate (and the default)
// K-split down ring depth: its items are two tiles, twice the weights of a
// claimed down item (3 measured best at 8 and 16 rows, against 4 and 5)
template <int FMT, int AL>
constexpr int ring_dn() { return 3; }
// claimed down ring depth (items of two tiles; 4 measured best at 64 rows, against 3)
template <int FMT, int AL>
constexpr int ring_dc() { return 4; }
// up/gate ring depth by activation loads per item (FP8 with 2 loads: 7
// measured best at 8 rows; MXFP4 with 2, whose items are two weight tiles:
// 3 measured best at 16 rows, against 4 and 5)
template <int FMT, int AL, bool W2 = false>
constexpr int ring_up() { return AL == 2 ? (FMT == 0 ? (W2 ? 6 : 7) : 3) : kRingD; }
template <int D = kRingD>
struct RingN {
  FetchN f;
  ItemN r[D];
  uint32_t aop[D], h2p[D];  // activation offsets of the filled items (split fill)
};

template <int FMT, int KIND, int D, int AL, bool W2 = false>
__device__ __forceinline__ void ring_open(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int k, int kend,
                                          bool& ok) {
  R.f.k = k;
  R.f.nch = 0;
  R.f.nu = -1;
  R.f.cnt = 0;
  R.f.ab = (const uint8_t*)(KIND == 1 ? arg_ptr(p.x) : arg_ptr(p.mid));
  fetch_next_any<FMT, KIND, AL, W2>(p, L, ph, R.f, kend, ok);
}

// WONLY: weights and scales only (the activation offsets are kept).
template <int FMT, int KIND, bool WONLY, int D, int AL, bool W2 = false>
__device__ __forceinline__ void ring_fill(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int kend,
                                          bool& ok) {
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (WONLY) {
      fetch_weights_n<FMT, item_wt<FMT, KIND, AL, W2>()>(R.f, R.r[d]);
      R.aop[d] = R.f.ao;
      R.h2p[d] = R.f.h2;
    } else {
      fetch_item_n<FMT, AL, item_wt<FMT, KIND, AL, W2>()>(R.f, R.r[d]);
    }
    fetch_adv_n<FMT>(R.f);
    if (R.f.left == 0) fetch_next_any<FMT, KIND, AL, W2>(p, L, ph, R.f, kend, ok);
  }
}

template <int FMT, int D, int AL>
__device__ __forceinline__ void ring_fill_acts(RingN<D>& R) {
#pragma unroll
  for (int d = 0; d < D; ++d) fetch_acts_n<FMT, AL>(R.f.ab, R.aop[d], R.h2p[d], R.r[d]);
}

// PEEL: the first round is its own copy, so that the loop's waits are
// counted from the steady load order (a split fill issues them in another).
// Up/gate (KIND 1): chunks are claimed from the CU's counter and chunk ends
// go through the partial windows.
template <int FMT, int KIND, bool PEEL, int D, int AL, bool W2 = false>
__device__ __forceinline__ void ring_run(const Params& p, const Lds& L, const PhaseN& ph, RingN<D>& R, int k, int kend,
                                         int& jc, bool& ok) {
  EatN e;
  e.k = k;
  e.nch = 0;
  const bool any = KIND == 1   ? eat_next_up<FMT, AL, W2>(p, L, ph, e, R.f.nch)
                   : KIND == 3 ? eat_next_dc<FMT, AL>(p, L, ph, e, R.f.nch)
                               : eat_next_n<FMT, KIND, AL>(p, L, ph, e, kend);
  if (any) {
    const int lg = (threadIdx.x & 63) >> 4;
    constexpr int WT = item_wt<FMT, KIND, AL, W2>();
    const int split_c = KIND == 3 ? 0 : ph_split<KIND, WT>(ph);
    const int split2_c = KIND == 3 ? 0 : ph_split2<KIND>(ph);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};  // a two-tile item's tile B
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};  // KIND 3: the unit's sum over its K-phases
    f32x4 tot2 = {0.f, 0.f, 0.f, 0.f};  // KIND 3: the same for its tile B
    // The loop is left only after a whole round of D slots: once the last
    // job has ended, the rest of the round multiplies dead items and
    // refills with dead loads.  So every path to an item's wait has issued
    // the same D-1 items since (an exit in mid-round would make the
    // compiler's wait counting assume fewer and drain the ring).
    bool done = false;
    auto round = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int split = KIND == 3 ? e.split : split_c;
        const int split2 = KIND == 3 ? e.split2 : split2_c;
        if (FMT == 0 || e.fmt == 0) eat_item_n<0, AL, WT, FMT != 0>(split, split2, lg, R.r[d], acc, acc2);
        else eat_item_n<1, AL, WT>(split, split2, lg, R.r[d], acc, acc2);
        fetch_item_n<FMT, AL, WT>(R.f, R.r[d]);
        fetch_adv_n<FMT>(R.f);
        if (R.f.left == 0) fetch_next_any<FMT, KIND, AL, W2>(p, L, ph, R.f, kend, ok);
        if (!done) {
          e.left = uni(e.left) - 1;
          if (KIND == 3 && e.left == 0) {
            bool unit_end;
            done = !dc_phase_end<FMT, AL>(p, L, ph, e, acc, tot, acc2, tot2, R.f.nch, unit_end);
            if (unit_end) {
              MOE_JSTAMP(p, jc);
              balance(L, ++jc);
            }
          } else if (e.left == 0) {
            if (KIND == 1) up_job_end<WT>(p, L, e, acc, acc2, ph.nw, ok);
            else if (e.pst) {
              lds_st128(L.pbuf + e.pidx, __builtin_bit_cast(u32x4, acc));
              if (WT == 2 && ph.nlive2 > 0) lds_st128(L.pbuf + e.pidx + 16, __builtin_bit_cast(u32x4, acc2));
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
            MOE_JSTAMP(p, jc);
            balance(L, ++jc);
            done = KIND == 1 ? !eat_next_up<FMT, AL, W2>(p, L, ph, e, R.f.nch)
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
// order, rounded to bf16 once.  Each product is first summed over the
// K-phases of its tile in order (sum_kphases).
__device__ __forceinline__ float down_product(const Params& p, const Lds& L, int r, int slot, int hl) {
  return L.pbuf[((size_t)r * (p.K + 1) + slot) * p.pitch + hl];  // summed by sum_kphases
}

// Each (row, slot, h) product is first summed over its K-phases (in order,
// into the K-phase 0 copy) by one thread per product, so the row's chain
// below reads one value per slot.  With one K-phase (claimed down jobs)
// there is nothing to sum: the combine checks the products.  Whole
// workgroup; ends synchronised.
template <bool ONE>
__device__ inline void sum_kphases(const Params& p, const Lds& L, const Sched& s) {
  if (ONE) return;
  const size_t kstride = (size_t)p.T * (p.K + 1) * p.pitch;
  const int n = p.T * (p.K + 1) * s.hc;
  for (int t = threadIdx.x; t < n; t += kThreads) {
    const int rs = t / s.hc, hl = t - rs * s.hc;  // rs = row * (K+1) + slot
    float* q = L.pbuf + (size_t)rs * p.pitch + hl;
    float c[kWaves];  // the copies read before the sum (wpt <= 8), in flight together
#pragma unroll
    for (int kp = 0; kp < kWaves; ++kp) c[kp] = kp < s.wpt ? q[kp * kstride] : 0.f;
    float v = 0.f;
#pragma unroll
    for (int kp = 0; kp < kWaves; ++kp)
      if (kp < s.wpt) v += c[kp];
    if (!isfinite(v)) set_err(p.err, kErrMid);
    q[0] = v;
  }
  __syncthreads();
}

// A pick whose expert is not held here (expert range) has no column: its
// product stays at the zeroed partials, and its term adds exactly +0.
// RES: a residual, when given, is added in fp32 after the chain, then
// rounded once (the residual add of the unfused layout, folded in).
// SHONLY: the shared expert's product alone (the unfused layout's shared
// down launch).
// ONE: one K-phase (claimed down jobs, wpt = 1), so nothing was summed
// before and the products are checked here; the picks' weights and
// products are then read before the chain (K <= 8), their LDS reads in
// flight together (a chain of dependent reads per row is the longer path
// at 64 rows).
template <bool RES, bool SHONLY = false, bool ONE = false>
__device__ inline void combine(const Params& p, const Lds& L, const Sched& s) {
  for (int t = threadIdx.x; t < p.T * s.hc; t += kThreads) {
    const int r = t / s.hc, hl = t - r * s.hc;
    const size_t o = (size_t)r * p.H + s.h0 + hl;
    const uint32_t res = RES && p.residual ? p.residual[o] : 0u;  // issued ahead of the chain
    float acc = p.n_shared ? down_product(p, L, r, p.K, hl) : 0.f;
    if (ONE) {
      bool bad = !isfinite(acc);
      if (!SHONLY) {
        float wv[kMaxTopK], pv[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
          wv[k] = k < p.K ? L.w[r * p.K + k] : 0.f;
          pv[k] = k < p.K ? down_product(p, L, r, k, hl) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
          if (k < p.K) acc = fmaf(wv[k], pv[k], acc);
          bad = bad || !isfinite(pv[k]);
        }
      }
      if (bad) set_err(p.err, kErrMid);
    } else if (!SHONLY) {
      for (int k = 0; k < p.K; ++k) acc = fmaf(L.w[r * p.K + k], down_product(p, L, r, k, hl), acc);
    }
    if (RES && p.residual) acc += bf16_bits_to_f32(res);
    p.out[o] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

// ------------------------------------------------------------------ kernel

__device__ __forceinline__ Sched make_sched(const Params& p, int G) {
  Sched s;
  s.sh_tiles = p.n_shared ? p.Is >> p.lti : 0;
  s.rt_tiles = p.I >> p.lti;
  s.G = G;
  s.n_pairs = s.sh_tiles + (G - p.n_shared) * s.rt_tiles;
  s.h0 = blockIdx.x * p.hs;
  s.hc = uni(p.H) - s.h0 < uni(p.hs) ? uni(p.H) - s.h0 : uni(p.hs);
  if (s.hc < 0) s.hc = 0;
  s.nrt = (s.hc + 15) / 16;
  s.nrt_p = uni(p.nrt_p);
  s.wpt = uni(p.wpt);
  s.kph = uni(p.kph);
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

// The forward after the logits: routing and grouping, the up/gate stream
// (its sums formed at job ends), the meeting (the call's one flag barrier), the down stream,
// the combine.  With at most as many rows as waves, the waves that route no
// row start on this CU's shared-expert jobs once every row's scores are in,
// the routing waves but wave 7 as soon as their row is routed, and wave 7
// once it has grouped the uses and written the routed tables.
// DCLAIM: down jobs claimed whole by the waves (above kKsplitRows rows),
// else split over the waves by K-phase.
// W2: FP8 up/gate items of two tiles (see stream_ti).
template <int FMT, int AL, bool DCLAIM, bool W2>
__device__ __forceinline__ void narrow_forward(char* smem, uint32_t epoch) {
  const int wave = wave_id();
  int jn = 0;  // jobs this wave has ended (for balance)
  bool ok = true;
  {
    constexpr int DU = ring_up<FMT, AL, W2>();
    RingN<DU> R;
    const Params& p = fresh_args();
    const Lds L = lds_map(smem, p);
    const int nkb = p.H / 128;
    PhaseN ph = {};
    ph.nw = nkb < kWaves ? nkb : kWaves;
    const int nS = shared_jobs_here(p);
    ph.nct = p.n_shared ? n_ctiles(p, p.T) : 1;
    ph.nsc = nS * ph.nw;
    const bool early = p.T <= kWaves && p.T * p.K <= 64 && nS > 0;
    const bool spread = nS > 0 && p.T >= kSpreadRows && (early || p.T > kWaves);
    MOE_STAMP(p, 2);
    if (spread) {
      // From 8 rows up each row is routed by wave 7 of one CU (row r: CU
      // r mod ncu), which publishes its picks; wave 7 of every CU then reads
      // every row's picks, groups the uses and writes the routed tables.
      // Waves 0..6 start on the CU's shared-expert chunks at once, except on
      // a CU that routes a row, where they wait until its scores are in.
      int here = 0;
      for (int r = (int)blockIdx.x; r < p.T; r += p.ncu) ++here;
      if (wave == kWaves - 1) {
        __builtin_amdgcn_s_setprio(3);
        for (int r = (int)blockIdx.x; r < p.T; r += p.ncu) route_publish(p, L, r, epoch + 1, 0);
        if (p.T * p.K <= 64) {
          read_picks<1>(p, L, epoch + 1, threadIdx.x & 63, 64);
          wave_sync();
          MOE_LSTAMP(p, 10);
          groups_one_wave<1>(p, L);
        } else {
          read_picks<kMaxRows * kMaxTopK / 64>(p, L, epoch + 1, threadIdx.x & 63, 64);
          wave_sync();
          MOE_LSTAMP(p, 10);
          groups_one_wave<kMaxRows * kMaxTopK / 64>(p, L);
        }
        wave_sync();
        MOE_LSTAMP(p, 3);
        const int G = lds_ldi_uniform(L.misc);
        const Sched s = make_sched(p, G);
        routed_tables<1>(p, L, s, nS);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the up/gate tables, before the flag
        lds_st32(L.misc + kMiscReady, 1u);
        routed_tables<2>(p, L, s, nS);
        __builtin_amdgcn_s_setprio(0);
        MOE_LSTAMP(p, 11);
      } else if (here > 0) {
        lds_wait<1>(p, (const uint32_t*)L.misc + kMiscPolled, (uint32_t)here, ok);
      }
    } else if (early) {
      // The top T waves route (row r by wave 7 - r; the scores of a batch
      // under 8 rows are published by wave 0), wave 7 then groups.  The
      // streaming waves start once every row's scores are in: their loads
      // would otherwise queue ahead of the polls.  The routing waves run at
      // raised priority until their rows are routed.
      const int r = kWaves - 1 - wave;
      if (r < p.T) {
        __builtin_amdgcn_s_setprio(3);
        route_row(p, L, r, epoch + 1, wave);
        if (r != 0) __builtin_amdgcn_s_setprio(0);
        lds_inc_lane0((uint32_t*)(L.misc + kMiscRouted));  // after this wave's ids / w writes (LDS order)
      }
      if (r == 0) {
        lds_wait<1>(p, (const uint32_t*)L.misc + kMiscRouted, (uint32_t)p.T, ok);
        MOE_LSTAMP(p, 10);
        groups_one_wave<1>(p, L);
        wave_sync();
        MOE_LSTAMP(p, 3);
        const int G = lds_ldi_uniform(L.misc);
        const Sched s = make_sched(p, G);
        routed_tables<1>(p, L, s, nS);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the up/gate tables, before the flag
        lds_st32(L.misc + kMiscReady, 1u);
        MOE_LSTAMP(p, 59);
        // the down tables are read after the phase barrier
        routed_tables<2>(p, L, s, nS);
        __builtin_amdgcn_s_setprio(0);
        MOE_LSTAMP(p, 11);
      }
      if (r >= p.T) lds_wait<1>(p, (const uint32_t*)L.misc + kMiscPolled, (uint32_t)p.T, ok);
    } else {
      if (p.T > kWaves) {
        route_rows_spread(p, L, epoch + 1);
      } else {
        for (int r = wave; r < p.T; r += kWaves) route_row(p, L, r, epoch + 1, wave);
      }
      __syncthreads();
      MOE_STAMP(p, 10);
      build_groups(p, L);
      MOE_STAMP(p, 3);
      const int G = lds_ldi_uniform(L.misc);
      const Sched s = make_sched(p, G);
      if (wave == 0) routed_tables<3>(p, L, s, nS);
      if (threadIdx.x == 0) L.misc[kMiscReady] = 1;
      __syncthreads();
      MOE_STAMP(p, 11);
    }
    ring_open<FMT, 1, DU, AL, W2>(p, L, ph, R, 0, nS, ok);
    MOE_STAMP(p, 62);
    ring_fill<FMT, 1, false, DU, AL, W2>(p, L, ph, R, nS, ok);
    MOE_STAMP(p, 13);
    ring_run<FMT, 1, false, DU, AL, W2>(p, L, ph, R, 0, nS, jn, ok);
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
    const int nD = lds_ldi_uniform(L.misc + kMiscND);
    const Sched s = make_sched(p, G);
    zero_partials(L, (size_t)p.wpt * p.T * (p.K + 1) * p.pitch);
    // the first D items' weights do not depend on mid: issue them before the
    // wait, their activations after it
    constexpr int DD = DCLAIM ? ring_dc<FMT, AL>() : ring_dn<FMT, AL>();
    RingN<DD> R;
    if (!DCLAIM) {
      // each wave takes its tiles of this CU's slice in one K-phase of the
      // down jobs it shares out with the other waves (see ksplit_phase)
      const PhaseN ph = ksplit_phase<item_wt<FMT, 2, AL>()>(p, s, wave);
      const int kend = ph.nlive > 0 ? p.qcap + nD : p.qcap;
      ring_open<FMT, 2, DD, AL>(p, L, ph, R, p.qcap, kend, ok);
      ring_fill<FMT, 2, true, DD, AL>(p, L, ph, R, kend, ok);
      wait_all(p, epoch + 2);
      MOE_STAMP(p, 5);
      MOE_WSTAMP(p, 1);
      ring_fill_acts<FMT, DD, AL>(R);
      ring_run<FMT, 2, true, DD, AL>(p, L, ph, R, p.qcap, kend, jn, ok);
    } else {
      // the waves claim (down job, pair of 16-row tiles) units and stream
      // all their K-blocks, K-phase by K-phase
      const PhaseN ph = down_phase(s.h0, s.hc, s.nrt, 0, 0, 31 - __builtin_clz(s.kph));
      const int nunits = s.hc > 0 ? nD * ((s.nrt + 1) >> 1) : 0;  // units: a job's pairs of 16-row tiles
      ring_open<FMT, 3, DD, AL>(p, L, ph, R, -1, nunits, ok);
      ring_fill<FMT, 3, true, DD, AL>(p, L, ph, R, nunits, ok);
      wait_all(p, epoch + 2);
      MOE_STAMP(p, 5);
      MOE_WSTAMP(p, 1);
      ring_fill_acts<FMT, DD, AL>(R);
      ring_run<FMT, 3, true, DD, AL>(p, L, ph, R, 0, nunits, jn, ok);
    }
    MOE_WSTAMP(p, 2);
    MOE_STAMP(p, 6);
  }
  {
    const Params& p = fresh_args();
    const Lds L = lds_map(smem, p);
    const Sched s = make_sched(p, G);
    __syncthreads();
    sum_kphases<DCLAIM>(p, L, s);
    combine<true, false, DCLAIM>(p, L, s);
    MOE_STAMP(p, 7);
#ifdef MOE_TIMELINE
    __syncthreads();
    if (threadIdx.x < 64 && p.timeline) p.timeline[blockIdx.x * 64 + threadIdx.x] = MOE_TL(p, threadIdx.x);
#endif
  }
}


// The unfused layout's shared-expert launches ("Daily AI Hotspot
// 2026-08-21", "Most Worth Your Attention Today": the shared expert's
// gate/up and its down are launches of their own between the routed MoE
// and the add), run by the same stream without routing: UP streams this
// CU's shared gate/up jobs and leaves mid in the workspace (visible to the
// next launch at the kernel boundary); otherwise the down jobs of the shared
// group read that mid, and the shared product alone is rounded to bf16.
template <int FMT, int AL, bool DCLAIM, bool UP, bool W2>
__device__ __forceinline__ void shared_only(char* smem) {
  const Params& p = fresh_args();
  const Lds L = lds_map(smem, p);
  const int wave = wave_id(), nS = shared_jobs_here(p);
  int jn = 0;
  bool ok = true;
  const Sched s = make_sched(p, 1);
  if (wave == 0) {
    if (UP) {
      if (threadIdx.x == 0) L.misc[kMiscNU] = nS;
    } else {
      routed_tables<2>(p, L, s, nS);
    }
  }
  if (threadIdx.x == 0) {
    L.misc[0] = 1;
    L.misc[kMiscReady] = 1;
  }
  __syncthreads();
  if (UP) {
    const int nkb = p.H / 128;
    PhaseN ph = {};
    ph.nw = nkb < kWaves ? nkb : kWaves;
    ph.nct = n_ctiles(p, p.T);
    ph.nsc = nS * ph.nw;
    constexpr int DU = ring_up<FMT, AL, W2>();
    RingN<DU> R;
    ring_open<FMT, 1, DU, AL, W2>(p, L, ph, R, 0, nS, ok);
    ring_fill<FMT, 1, false, DU, AL, W2>(p, L, ph, R, nS, ok);
    ring_run<FMT, 1, false, DU, AL, W2>(p, L, ph, R, 0, nS, jn, ok);
    return;
  }
  const int nD = lds_ldi_uniform(L.misc + kMiscND);
  zero_partials(L, (size_t)p.wpt * p.T * (p.K + 1) * p.pitch);
  __syncthreads();
  constexpr int DD = DCLAIM ? ring_dc<FMT, AL>() : ring_dn<FMT, AL>();
  RingN<DD> R;
  if (!DCLAIM) {
    const PhaseN ph = ksplit_phase<item_wt<FMT, 2, AL>()>(p, s, wave);
    const int kend = ph.nlive > 0 ? p.qcap + nD : p.qcap;
    ring_open<FMT, 2, DD, AL>(p, L, ph, R, p.qcap, kend, ok);
    ring_fill<FMT, 2, false, DD, AL>(p, L, ph, R, kend, ok);
    ring_run<FMT, 2, false, DD, AL>(p, L, ph, R, p.qcap, kend, jn, ok);
  } else {
    const PhaseN ph = down_phase(s.h0, s.hc, s.nrt, 0, 0, 31 - __builtin_clz(s.kph));
    const int nunits = s.hc > 0 ? nD * ((s.nrt + 1) >> 1) : 0;  // units: a job's pairs of 16-row tiles
    ring_open<FMT, 3, DD, AL>(p, L, ph, R, -1, nunits, ok);
    ring_fill<FMT, 3, false, DD, AL>(p, L, ph, R, nunits, ok);
    ring_run<FMT, 3, false, DD, AL>(p, L, ph, R, 0, nunits, jn, ok);
  }
  __syncthreads();
  sum_kphases<DCLAIM>(p, L, s);
  combine<false, true, DCLAIM>(p, L, s);
}

// A forward after an upstream producer (moe_forward_after): each wave first
// issues loads of weights that do not depend on x, its piece of this CU's
// router row and of the first item of the CU's first shared-expert job, so
// they reach the caches while the producer finishes; then it polls the
// ready word (agent scope, bounded: on timeout the error bit is set and the
// call runs on), then acquires at agent scope before any load of x.
__device__ inline void wait_x_ready(const Params& p) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if ((int)blockIdx.x < p.E) {
    const int ch = p.H / kWaves, ngrp = ch >> 3;
    a = ld16(p.router_w + (size_t)blockIdx.x * p.H + (size_t)wave * ch + 8 * (lane < ngrp ? lane : ngrp - 1));
  }
  if (p.n_shared && (int)blockIdx.x < (p.Is >> p.lti) && wave < p.H / 128) {
    const int row = lane & 15, t = blockIdx.x;
    const int lrow = p.lti == 4 ? 16 * t + row : row < 8 ? 8 * t + row : p.Is + 8 * t + row - 8;
    b = ld16(p.sh_wgu + (size_t)lrow * p.H + 128 * wave + 32 * (lane >> 4));
  }
  for (uint32_t spins = 0;;) {
    const uint32_t v = __hip_atomic_load(p.x_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int32_t)(v - p.x_ready_value) >= 0) break;
    if (++spins > p.x_spins) {
      if (lane == 0) set_err(p.err, kErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::"v"(a), "v"(b));  // (the early loads are complete by now)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// NARROW picks the stream by batch size (see stream_al): 2 for one
// activation load per item, 3 for two (down jobs split over the waves by
// K-phase), 4 above kKsplitRows rows (two loads, down jobs claimed whole).
// The routing-only modes are instantiated with 1.
template <int MODE, int FMT, int NARROW>
__global__ __launch_bounds__(kThreads, 1) void moe_fused(Params p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Lds L = lds_map(smem, p);
  const int tid = threadIdx.x, wave = wave_id();

#ifdef MOE_TIMELINE
  if (tid > 0 && tid < 64) MOE_TL(p, tid) = 0;  // stamps this call does not take stay zero
#endif
  MOE_STAMP(p, 0);
  if (MODE == kModeSharedUp || MODE == kModeSharedDown) {
    if (tid < 64) L.ctl[tid] = 0u;
    stream_init(p, L, shared_jobs_here(p));
    __syncthreads();
    constexpr int AL = NARROW == 2 ? 1 : 2;
    shared_only<FMT, AL, NARROW >= 4, MODE == kModeSharedUp, NARROW == 4>(smem);
    return;
  }
  if (MODE == kModeForward) {
    // Every wave reads the epoch for itself and first needs it to tag its
    // scores, after the router loads have come in.  The stream's LDS words
    // are set before the first meeting.  The scores are read through their
    // tags, so no flag is raised after them (waiting for the score stores
    // to reach memory would hold the workgroup for a store round trip).
    const uint32_t ep = __hip_atomic_load(&p.flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 64) L.ctl[tid] = 0u;
    stream_init(p, L, shared_jobs_here(p));
    __syncthreads();
    if (p.x_ready) wait_x_ready(p);
    if (p.T < kWaves) {
      router_logits(p, L, ep, 1u);
      // the logit partials lie in wave 0's routing scratch (wave 0 reads
      // them) unless the experts are few
      const int nd = (p.E > (int)blockIdx.x ? (p.E - 1 - (int)blockIdx.x) / p.ncu + 1 : 0) * p.T;
      if (kWaves * nd > p.E) __syncthreads();
    } else {
      router_logits_rows<true>(p, ep);
    }
    MOE_STAMP(p, 1);
    constexpr int AL = NARROW == 2 ? 1 : 2;
    narrow_forward<FMT, AL, NARROW >= 4, NARROW == 4>(smem, __builtin_amdgcn_readfirstlane(ep));
    return;
  }

  // The routing-only calls: logits of this CU's experts published for
  // every CU, then workgroup 0 routes every row (polling the tagged score
  // slots) and groups the step's distinct experts.
  if (tid < 64) L.ctl[tid] = 0u;
  if (tid == 0)
    L.misc[1] = (int32_t)__hip_atomic_load(&p.flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t epoch = (uint32_t)__builtin_amdgcn_readfirstlane(L.misc[1]);
  if (p.T < kWaves) router_logits(p, L, epoch, 1u);
  else router_logits_rows<false>(p, epoch + 1);
  publish(p, epoch + 1);
  MOE_STAMP(p, 1);
  if (blockIdx.x != 0) return;
  MOE_STAMP(p, 2);
  for (int r = wave; r < p.T; r += kWaves) route_row(p, L, r, epoch + 1, wave);
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
}

// ------------------------------------------------------------------ host glue

WsLayout ws_layout(int max_rows, int E, int K, int H, int I, int Is) {
  (void)H;
  WsLayout w;
  size_t q = 0;
  w.flags = q; q = align_up(q + 4 * 1024, 256);
  w.err = q; q = align_up(q + 256, 256);
  w.scores = q; q = align_up(q + 16 * (size_t)max_rows * 4 * ((E + 3) / 4), 256);
  w.picks = q; q = align_up(q + 16 * (size_t)max_rows * K, 256);
  w.mid_ld = (I > Is ? I : Is);
  w.mid = q; q = align_up(q + 2 * (size_t)max_rows * (K + 1) * w.mid_ld, 256);
  w.total = q;
  return w;
}

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

template <int MODE, int FMT>
static hipError_t launch_forward(const Params& p, hipStream_t stream, int dev) {
  // above kKsplitRows rows: two-tile up/gate items (4) or, for an FP8 layer
  // whose tiles are 8 intermediates (stream_geometry), one-tile items (5)
  if (p.T > kKsplitRows)
    return FMT == 0 && p.ti == 8 ? launch_one<MODE, FMT, 5>(p, stream, dev) : launch_one<MODE, FMT, 4>(p, stream, dev);
  return stream_al(p.T) == 1 ? launch_one<MODE, FMT, 2>(p, stream, dev) : launch_one<MODE, FMT, 3>(p, stream, dev);
}

hipError_t launch(const Params& p, int mode, hipStream_t stream, int dev) {
  if (mode == kModeForward)
    return p.routed_fmt == 0 ? launch_forward<kModeForward, 0>(p, stream, dev)
                             : launch_forward<kModeForward, 1>(p, stream, dev);
  // the shared expert is FP8 in every format
  if (mode == kModeSharedUp) return launch_forward<kModeSharedUp, 0>(p, stream, dev);
  if (mode == kModeSharedDown) return launch_forward<kModeSharedDown, 0>(p, stream, dev);
  if (mode == kModeRoute) return launch_one<kModeRoute, 0>(p, stream, dev);
  return launch_one<kModeGroups, 0>(p, stream, dev);
}

__global__ void add_bf16(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, uint16_t* __restrict__ out,
                         size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = (uint16_t)f32_to_bf16_rne(bf16_bits_to_f32(a[i]) + bf16_bits_to_f32(b[i]));
}

hipError_t launch_add(const uint16_t* a, const uint16_t* b, uint16_t* out, size_t n, hipStream_t stream) {
  const size_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(add_bf16, dim3((unsigned)(blocks ? blocks : 1)), dim3(256), 0, stream, a, b, out, n);
  return hipGetLastError();
}

}  // namespace moe
