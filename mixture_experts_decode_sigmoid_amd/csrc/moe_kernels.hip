// moe_kernels.hip -- the fused decode MoE pass for MI355X (gfx950, CDNA4).
//
// One persistent launch: one workgroup of 8 waves per CU, all resident.
//
//   S0  router logits   CU c computes l[r][e] for its experts e = c, c+ncu..
//                       (fp64 sums of exact bf16 products), sigmoid, bias;
//                       publishes them, then raises its flag (epoch + 1).
//   S1  shared up/gate  the shared expert does not depend on routing, so its
//                       8-intermediate tiles are streamed while the other CUs
//                       finish S0.
//   S2  route + group   every CU waits for all flags, routes every row itself
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
// Cross-CU data (scores, mid) is published with an agent-scope release fence
// before a flag store and read after polling the flags and an agent-scope
// acquire fence.  Each CU owns one flag and raises it by one per phase; a
// call advances every flag by two, so the workspace needs no reset.  Waits
// are bounded: on timeout an error bit is set and the kernel runs on.
#include "moe_internal.h"

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

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// Optional per-CU phase stamps (build with -DMOE_TIMELINE): thread 0 of each
// workgroup writes s_memrealtime (100 MHz) at phase boundaries into
// p.timeline[blockIdx.x * 16 + i].
#ifdef MOE_TIMELINE
#define MOE_STAMP(p, i)                                                                  \
  do {                                                                                   \
    if (threadIdx.x == 0 && (p).timeline)                                                \
      (p).timeline[blockIdx.x * 16 + (i)] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#else
#define MOE_STAMP(p, i) \
  do {                  \
  } while (0)
#endif

// ------------------------------------------------------------------ LDS map

// Weight stages: a ring of `ns` stages, each 16 weight rows of one K chunk
// (1024 elements: 1024 B of FP8 or 512 B of MXFP4) in slots of 1040 B.  A
// DMA instruction always writes 64 lanes x 16 B = 1 KB, so each row owns a
// full 1 KB slot (an MXFP4 row's second half holds filler nobody reads); the
// 16-byte pad puts the 16 rows an MFMA tile reads in one ds_read_b128 on
// different LDS banks.
constexpr int kPitch = 1040;
constexpr int kStageBytes = 16 * kPitch;
constexpr int kChunkElems = 1024;

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
  int32_t* misc;     // [32]: 0 = G, 1 = epoch, 8.. = scan
  uint32_t* ctl;     // [64] chunk-stream counters (see kCtl*)
  float* red;        // [red_slots][red_tiles][kWaves][64][4] job-end partials
  double* rb;        // [kWaves][E] router keys (aliases red and pbuf)
  double* rgs;       // [kWaves][64] group scores
  int32_t* rkept;    // [kWaves][64]
  float* pbuf;       // [T*(K+1)][hs] down products (batches of at most 16 rows)
  char* stages;      // [ns][kStageBytes]
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Job-end partials: up to 16 columns per tile when a batch has at most 16
// rows (one tile, two slots), else 4 tiles in one slot.
__host__ __device__ inline int red_tiles(int T) { return T > 16 ? kMaxRows / 16 : 1; }
__host__ __device__ inline int red_slots(int T) { return T > 16 ? 1 : 2; }
constexpr size_t kRedTileBytes = 16 * (size_t)kWaves * 64;  // one tile: [wave][lane] f32x4

struct LdsOffsets {
  size_t ids, w, first, egrp, rmask, gexp, gcnt, gstart, cols, misc, ctl, red, pbuf, stages;
};

__host__ __device__ inline LdsOffsets lds_offsets(int T, int K, int E, int hs) {
  LdsOffsets o;
  size_t q = 0;
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
  o.misc = q; q = align_up(q + 4 * 32, 16);
  o.ctl = q; q = align_up(q + 4 * 64, 16);
  // the routing scratch (used before the stream) overlaps the job-end
  // partials and the down products (used in it)
  o.red = q;
  const size_t rd = (size_t)red_slots(T) * red_tiles(T) * kRedTileBytes;
  o.pbuf = q + rd;
  const size_t pb = T > kLdsProdRows ? 0 : 4 * (size_t)T * (K + 1) * hs;
  const size_t rs = 8 * (size_t)kWaves * E + 8 * (size_t)kWaves * 64 + 4 * (size_t)kWaves * 64;
  q = align_up(q + (rd + pb > rs ? rd + pb : rs), 16);
  o.stages = q;
  return o;
}

size_t lds_plan(int T, int K, int E, int hs, size_t max_lds, int* ns) {
  const size_t fixed = lds_offsets(T, K, E, hs).stages;
  if (fixed + 2 * (size_t)kStageBytes > max_lds) {
    *ns = 0;
    return fixed + 2 * (size_t)kStageBytes;
  }
  size_t n = (max_lds - fixed) / kStageBytes;
  if (n > 8) n = 8;
  *ns = (int)n;
  return fixed + n * kStageBytes;
}

__device__ inline Lds lds_map(char* base, const Params& p) {
  LdsOffsets o = lds_offsets(p.T, p.K, p.E, p.hs);
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
  L.misc = (int32_t*)(base + o.misc);
  L.ctl = (uint32_t*)(base + o.ctl);
  L.red = (float*)(base + o.red);
  L.pbuf = (float*)(base + o.pbuf);
  L.rb = (double*)(base + o.red);
  L.rgs = L.rb + (size_t)kWaves * p.E;
  L.rkept = (int32_t*)(L.rgs + (size_t)kWaves * 64);
  L.stages = base + o.stages;
  return L;
}

// ------------------------------------------------------------------ flags

// Raise this CU's flag to `value` after all of the workgroup's prior global
// stores.  Every compute wave waits for its own stores, the workgroup meets,
// then one thread releases at agent scope and stores the flag.  The barrier
// is the bare s_barrier: producer waves may have weight DMA in flight and
// must not wait for it here.
__device__ inline void publish(const Params& p, uint32_t value) {
  if ((threadIdx.x >> 6) < kWaves) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(&p.flags[blockIdx.x], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until every CU's flag has reached `target` (wrap-around safe), then
// acquire.  Wave 0 polls and acquires; the barrier after it orders the rest
// of the workgroup (bare s_barrier, as in publish).
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

__device__ inline void wait_all(const Params& p, uint32_t target) {
  if (threadIdx.x < 64) poll_flags(p, target);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ S0 logits

__device__ inline double load_bias(const Params& p, int e) {
  if (p.bias_bf16) return (double)bf16_bits_to_f32(((const uint16_t*)p.bias)[e]);
  return (double)((const float*)p.bias)[e];
}

// l[r][e] = sum_h x[r][h] * Wr[e][h]: lane l sums h = 8l + 512j + 0..7 in
// order, then a fixed xor butterfly; one wave per (row, expert).  The loads
// of up to 8 j are issued before their products are summed.
__device__ inline void router_logits(const Params& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= kWaves) return;
  for (int e = blockIdx.x; e < p.E; e += p.ncu) {
    const uint16_t* wr = p.router_w + (size_t)e * p.H;
    const double bias = load_bias(p, e);
    for (int r = wave; r < p.T; r += kWaves) {
      const uint16_t* xr = p.x + (size_t)r * p.H;
      double acc = 0.0;
      for (int h0 = 8 * lane; h0 < p.H; h0 += 512 * 8) {
        u32x4 xv[8], wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int h = h0 + 512 * j < p.H ? h0 + 512 * j : h0;
          xv[j] = ld16(xr + h);
          wv[j] = ld16(wr + h);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (h0 + 512 * j < p.H) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t xa = xv[j][i], wa = wv[j][i];
              acc = fma((double)bf16_bits_to_f32(xa & 0xffffu), (double)bf16_bits_to_f32(wa & 0xffffu), acc);
              acc = fma((double)bf16_bits_to_f32(xa >> 16), (double)bf16_bits_to_f32(wa >> 16), acc);
            }
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (lane == 0) {
        double s = 1.0 / (1.0 + exp(-acc));
        double b = s + bias;
        if (!isfinite(acc) || !isfinite(b)) set_err(p.err, kErrScore);
        double* dst = p.scores + ((size_t)r * p.E + e) * 2;
        dst[0] = s;
        dst[1] = b;
      }
    }
  }
}

// ------------------------------------------------------------------ S2 routing

__device__ __forceinline__ bool key_before(double b1, int e1, double b2, int e2) {
  return b1 > b2 || (b1 == b2 && e1 < e2);
}

// Routes row r with one wave: group stage (sum of the two best keys per
// group, keep k_g groups by (score desc, index asc)), then K rounds of wave
// argmax over (key desc, index asc); weights s/sum(s)*scale in fp64.
__device__ inline void route_row(const Params& p, const Lds& L, int r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double* sc = p.scores + (size_t)r * p.E * 2;
  double bv[4], sv[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    alive[i] = e < p.E;
    double b = alive[i] ? sc[2 * e + 1] : -INFINITY;
    sv[i] = alive[i] ? sc[2 * e] : 0.0;
    bv[i] = isnan(b) ? -INFINITY : b;
  }
  if (p.ng > 1) {
    double* rb = L.rb + (size_t)wave * p.E;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (alive[i]) rb[lane + 64 * i] = bv[i];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int gsz = p.E / p.ng;
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
  double ssum = 0.0;
  int picks[kMaxTopK];
  double pick_s[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < p.K) {
      double bb = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (alive[i] && key_before(bv[i], e, bb, be)) { bb = bv[i]; be = e; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        double ob = __shfl_xor(bb, off, 64);
        int oe = __shfl_xor(be, off, 64);
        if (key_before(ob, oe, bb, be)) { bb = ob; be = oe; }
      }
      // be is now the same in every lane; its owner retires it
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == be) alive[i] = false;
      // the pick's score s, from the lane that holds it
      const int slot = be >> 6;
      const double mine = slot == 0 ? sv[0] : slot == 1 ? sv[1] : slot == 2 ? sv[2] : sv[3];
      const double sp = __shfl(mine, be & 63, 64);
      picks[k] = be;
      pick_s[k] = sp;
      ssum += sp;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (k < p.K) {
        L.ids[r * p.K + k] = picks[k];
        L.w[r * p.K + k] = (float)(pick_s[k] / ssum * p.routed_scale);
      }
    }
  }
}

// ------------------------------------------------------------------ S2 grouping

// Distinct experts of the step in order of first use over u = r*K + slot
// (group 0 = shared expert when present), each group's columns in ascending
// u.  Needs L.ids; whole workgroup; ends synchronised.
__device__ inline void build_groups(const Params& p, const Lds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = p.T * p.K;
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
  if (tid == 0) {
    L.misc[0] = G;
    int s = 0;
    if (p.n_shared) {
      L.gexp[0] = -1;
      L.gcnt[0] = p.T;
      L.gstart[0] = 0;
      s = p.T;
    }
    for (int g = p.n_shared; g < G; ++g) {
      L.gstart[g] = s;
      s += L.gcnt[g];
    }
  }
  __syncthreads();
  if (p.n_shared)
    for (int r = tid; r < p.T; r += kThreads) L.cols[r] = r * 16 + p.K;
  for (int u = tid; u < U; u += kThreads) {
    const int e = L.ids[u], r = u / p.K, slot = u - r * p.K;
    const uint32_t lo = L.rmask[2 * e], hi = L.rmask[2 * e + 1];
    const int rank = (r < 32) ? __popc(lo & ((1u << r) - 1u))
                              : __popc(lo) + __popc(hi & ((1u << (r - 32)) - 1u));
    const int g = L.egrp[e];
    L.cols[L.gstart[g] + rank] = r * 16 + slot;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ chunk stream
//
// Each CU streams a sequence of weight chunks: its shared-expert up/gate
// jobs, its routed up/gate jobs, then its down units.  A chunk is 16 weight
// rows x 1024 elements of the reduction axis.  Waves load chunks straight
// into an LDS ring (global_load_lds, 1 KB of one row per instruction, two
// rows per wave) `ns - 1` chunks ahead of the one being multiplied; wave w
// multiplies the 128-element K-block w of each chunk.  The activations
// (x for up/gate, mid for down) are loaded into registers one chunk ahead,
// always before that step's DMA, so the in-order vmcnt wait for them never
// waits for a newer DMA.

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Wave-uniform loop state, re-asserted as uniform: the compiler's uniformity
// analysis loses track of it across the stream loops (asm results, loop
// exits), and then keeps it in vector registers behind masked branches.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One row segment of up to 1 KB into LDS: 64 lanes x 16 B through a buffer
// resource whose size is the segment's valid bytes, so lanes past the end
// (a ragged tail, or a row with no valid bytes) read zeros without touching
// memory.  The buffer form of the LDS DMA is the one the compiler counts
// among outstanding vector memory operations.
__device__ __forceinline__ const void* uniform_ptr(const void* q) {
  const uint64_t v = (uint64_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// The descriptor's base and size are wave-uniform by construction; taking
// them through readfirstlane keeps the descriptor in scalar registers (a
// descriptor the compiler believes divergent costs a loop per instruction).
__device__ __forceinline__ void dma_row(const uint8_t* base, int nbytes, lds_char* l) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(base), 0,
                                                               __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16,
                                           (threadIdx.x & 63) * 16, 0, 0, 0);
}

// Waits until at most n of this wave's vector memory operations are
// outstanding (n is a multiple of 8: a producer issues 8 DMAs per chunk and
// keeps at most 7 chunks in flight, 56 operations, within the counter's 63).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
  }
}

// Workgroup barrier for LDS traffic only.  It does not wait for the weight
// DMA still in flight (a __syncthreads() would: its workgroup fence covers
// the DMA's LDS writes); DMA completion is awaited explicitly with wait_vm.
__device__ __forceinline__ void bar_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS accesses inside the chunk stream go through these: the compiler cannot
// tell them apart from the stage a DMA is still writing and would otherwise
// wait for every outstanding DMA (vmcnt(0)) before each of them.  Every block
// waits for its own LDS operation, so no asm load leaves a register in flight.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(size_t)(const lds_char*)p;
}
__device__ __forceinline__ uint32_t lds_off(const lds_char* p) { return (uint32_t)(size_t)p; }
template <class P>
__device__ __forceinline__ uint32_t lds_ld32(P p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
  return v;
}
template <class P>
__device__ __forceinline__ float lds_ldf(P p) { return __uint_as_float(lds_ld32(p)); }
// For an address every lane of the wave shares.
__device__ __forceinline__ int lds_ldi_uniform(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane((int)lds_ld32(p));
}
// Stores are not waited for: a wave's LDS operations complete in order, so
// a later flag store is seen after the data it publishes, and every reader
// waits for its own reads.  (A compiler-placed lgkmcnt wait that follows
// stays sufficient: an extra older operation completes first.)
__device__ __forceinline__ void lds_st32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st128(void* p, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
// Chunk-stream counters in LDS.  Every counter counts up from 0 within a
// launch and is written by one wave only.
constexpr int kCtlReady = 0;   // [2]  chunks producer pw has landed in LDS
constexpr int kCtlDone = 8;    // [8]  chunks compute wave w has finished reading
constexpr int kCtlPart = 16;   // [8]  jobs whose partials wave w has stored
constexpr int kCtlSlot = 24;   // [2]  1 + the last job summed out of partial slot s
constexpr int kCtlMidOut = 40; // [8]  1 once wave w's mid stores are complete
constexpr int kCtlCrossed = 48;// [1]  1 once wave 0 has seen every CU's mid

// Minimum of N consecutive LDS counters (N = 1, 2 or 8), one round trip.
// Every lane reads the same words; the result is taken through
// readfirstlane so the compiler knows it is uniform (an asm result is
// otherwise assumed divergent, and every branch on it becomes a masked one).
template <int N>
__device__ __forceinline__ uint32_t lds_min(const uint32_t* a) {
  if (N == 1) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(a)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
  } else if (N == 2) {
    uint64_t v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(a)) : "memory");
    const uint32_t v0 = (uint32_t)v, v1 = (uint32_t)(v >> 32);
    return __builtin_amdgcn_readfirstlane(v0 < v1 ? v0 : v1);
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

// A lane's part of one K-block of the stage, in one round trip: FP8, 32
// weight bytes; MXFP4, 16.
template <class P>
__device__ __forceinline__ void lds_ld_fp8_block(P w, u32x4& a, u32x4& b) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"(lds_off(w))
               : "memory");
}
template <class P>
__device__ __forceinline__ void lds_ld_fp4_block(P w, u32x4& a) {
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(a) : "v"(lds_off(w)) : "memory");
}

// LDS partials of a cross-wave reduction: wave w's f32x4 of lane l at
// red[(w*64 + l)*4 ..], so one lane's eight partials sit 1 KB apart.  These
// read a thread's 8 (down) or 2 x 8 (up/gate: gate at +0, up at +512 B)
// partials in one round trip.
__device__ __forceinline__ void lds_ld_partials8(const float* p, float (&a)[8]) {
  asm volatile(
      "ds_read_b32 %0, %8\n\tds_read_b32 %1, %8 offset:1024\n\t"
      "ds_read_b32 %2, %8 offset:2048\n\tds_read_b32 %3, %8 offset:3072\n\t"
      "ds_read_b32 %4, %8 offset:4096\n\tds_read_b32 %5, %8 offset:5120\n\t"
      "ds_read_b32 %6, %8 offset:6144\n\tds_read_b32 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(lds_off(p))
      : "memory");
}
__device__ __forceinline__ void lds_ld_partials16(const float* p, float (&a)[8], float (&b)[8]) {
  asm volatile(
      "ds_read_b32 %0, %16\n\tds_read_b32 %1, %16 offset:1024\n\t"
      "ds_read_b32 %2, %16 offset:2048\n\tds_read_b32 %3, %16 offset:3072\n\t"
      "ds_read_b32 %4, %16 offset:4096\n\tds_read_b32 %5, %16 offset:5120\n\t"
      "ds_read_b32 %6, %16 offset:6144\n\tds_read_b32 %7, %16 offset:7168\n\t"
      "ds_read_b32 %8, %16 offset:512\n\tds_read_b32 %9, %16 offset:1536\n\t"
      "ds_read_b32 %10, %16 offset:2560\n\tds_read_b32 %11, %16 offset:3584\n\t"
      "ds_read_b32 %12, %16 offset:4608\n\tds_read_b32 %13, %16 offset:5632\n\t"
      "ds_read_b32 %14, %16 offset:6656\n\tds_read_b32 %15, %16 offset:7680\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7]),
        "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7])
      : "v"(lds_off(p))
      : "memory");
}

// Column tiles a group can have: 1 when NPRE is 1 (batches of at most 16
// rows), else up to 4 (64 rows).
template <int NPRE>
constexpr int max_tiles() { return NPRE == 1 ? 1 : kMaxRows / 16; }

// Per-lane prefetch of one chunk: the activations of column tiles
// 0..NPRE-1; later tiles are loaded when used.
template <int NPRE>
struct Pre {
  u32x4 B[4 * NPRE];
  uint32_t sw;  // MXFP4: this lane's row's four E8M0 scales of its K-block
};

struct Sched {
  int sh_tiles;  // shared up/gate jobs (I_s / 8)
  int rt_tiles;  // routed up/gate jobs per group (I / 8)
  int n_jobs;    // all up/gate jobs, known after routing
  int G;         // groups, known after routing
  int h0, hc;    // this CU's down rows
  int nrt;       // 16-row tiles of them
  int routed;
};

// Position in this CU's job sequence.  A job is one up/gate tile of a group
// (8 gate + 8 up rows of W_gate_up over all of H) or one 16-row tile of this
// CU's down rows for a group (over the group's intermediate size); it is
// streamed as nchunks(K) chunks.
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

__device__ __forceinline__ int nchunks(int kdim) { return (kdim + kChunkElems - 1) / kChunkElems; }

// Smallest j >= begin with j = blockIdx.x (mod ncu): jobs are dealt round-robin.
__device__ __forceinline__ int first_job(const Params& p, int begin) {
  const int r = begin % p.ncu;
  return begin + (((int)blockIdx.x - r) % p.ncu + p.ncu) % p.ncu;
}

__device__ __forceinline__ bool blocked(const Sched& s, const It& c) {
  return c.phase == 0 && c.j >= s.sh_tiles;  // routed work before routing is known
}

// Up/gate jobs: the shared expert's tiles come first, then rt_tiles tiles
// per routed group; a down job names its group.  The group and tile are
// derived once on entering a phase and then advanced incrementally.
__device__ inline void settle(const Params& p, const Sched& s, It& c) {
  for (;;) {
    if (c.phase == 0) {
      c.g = 0;
      c.tile = c.j;
      if (c.j < s.sh_tiles || !s.routed) return;
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
      c.rt = 0;
      c.tile = 0;
      continue;
    }
    c.g = c.j;
    if (c.phase == 2 && (s.nrt <= 0 || c.j >= s.G)) c.phase = 3;
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
  } else if (++c.rt >= s.nrt) {
    c.rt = 0;
    ++c.j;
  }
  settle(p, s, c);
}

__device__ __forceinline__ int job_group(const Params&, const Sched&, const It& c) { return c.g; }
__device__ __forceinline__ int job_tile(const Sched&, const It& c) { return c.phase <= 1 ? c.tile : 0; }
__device__ __forceinline__ bool shared_group(const Params& p, int g) { return p.n_shared && g == 0; }
__device__ __forceinline__ int job_kdim(const Params& p, const It& c, int g) {
  return c.phase <= 1 ? p.H : (shared_group(p, g) ? p.Is : p.I);
}
__device__ __forceinline__ int group_ncols(const Params& p, const Lds& L, int g) {
  if (shared_group(p, g)) return p.T;
  return lds_ldi_uniform(L.gcnt + g);
}
// Column c of group g as row*16 + slot.
__device__ __forceinline__ int col_code(const Params& p, const Lds& L, int g, int c) {
  if (shared_group(p, g)) return c * 16 + p.K;
  return (int)lds_ld32(L.cols + lds_ldi_uniform(L.gstart + g) + c);
}

// ---------------------------------------------------------------- producers

// A producer wave's view of the job it streams: its 8 chunk rows (rows
// 8pw..8pw+7: gate rows 8t.., up rows I+8t.., or output rows) are
// consecutive rows of the weight matrix, so one base pointer and the row
// pitch address them; its lanes' part of the chunk's scale DMA is an offset
// that moves by 32 bytes per chunk.  Computed once per job.
struct Feed {
  It it;
  int kc, nck;
  const uint8_t* w;    // first of this wave's rows at K offset 0
  int rowbytes;        // bytes of one weight row
  int cbytes;          // bytes of one row per chunk
  int nl;              // live rows among this wave's 8 (may be <= 0)
};

__device__ inline void feed_job(const Params& p, const Lds& L, const Sched& s, Feed& f, int pw) {
  const It& c = f.it;
  const int g = job_group(p, s, c);
  const bool sh = shared_group(p, g), down = c.phase == 2;
  const int fmt = sh ? 0 : p.routed_fmt;
  const int iexp = sh ? p.Is : p.I;
  const int kdim = down ? iexp : p.H;
  const int tile = job_tile(s, c);
  const int hb = s.h0 + 16 * c.rt;
  const int nlive = down ? (s.hc - 16 * c.rt < 16 ? s.hc - 16 * c.rt : 16) : 16;
  const uint8_t* w;
  if (sh) {
    w = down ? p.sh_wd : p.sh_wgu;
  } else {
    // W_gate_up [E][2I][H], W_down [E][H][I] bytes (MXFP4: [E][2I][H/2], [E][H][I/2])
    const size_t e = (size_t)lds_ldi_uniform(L.gexp + g);
    const size_t H = p.H, I = p.I, div = fmt ? 2 : 1;
    w = down ? p.wd + e * H * (I / div) : p.wgu + e * 2 * I * (H / div);
  }
  f.kc = 0;
  f.nck = nchunks(kdim);
  f.rowbytes = fmt ? kdim / 2 : kdim;
  f.cbytes = fmt ? kChunkElems / 2 : kChunkElems;
  f.nl = nlive - 8 * pw;
  // a wave with no live rows keeps a valid base (it loads no bytes)
  const int row0 = down ? hb + (f.nl > 0 ? 8 * pw : 0) : (pw == 0 ? 8 * tile : iexp + 8 * tile);
  f.w = w + (size_t)row0 * f.rowbytes;
}

// Issues chunk f.kc of the job into `stage`: this wave's 8 row DMAs, always
// issued (a row past the live rows loads no bytes), so its vmcnt
// bookkeeping is 8 per chunk.
__device__ inline void feed_chunk(const Feed& f, lds_char* stage, int pw) {
  const int rb = __builtin_amdgcn_readfirstlane(f.rowbytes);
  const int cb = __builtin_amdgcn_readfirstlane(f.cbytes);
  const int koff = __builtin_amdgcn_readfirstlane(f.kc) * cb;
  const int nbytes = rb - koff < cb ? rb - koff : cb;
  const int nl = __builtin_amdgcn_readfirstlane(f.nl);
  const uint8_t* b = (const uint8_t*)uniform_ptr(f.w) + koff;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    dma_row(q < nl ? b + q * rb : b, q < nl ? nbytes : 0, stage + (8 * pw + q) * kPitch);
}

// ---------------------------------------------------------------- compute

// A compute wave's view of the job it multiplies, computed once per job.
template <int NPRE>
struct Eat {
  It it;
  int kc, nck;
  int kind;     // 1 up/gate, 2 down
  int g, tile, rt, fmt, kdim, nlive, ncols, nct;
  int eid;      // routed expert of the group
  int split;    // FP8: MFMA output rows (4*lg + q) below it take the first block scale
  float sreg;   // FP8: lane i < 32 holds the first row block's scale of K-block 8i + wave,
                // lane 32 + i the second block's (one load per job; read back by readlane)
  const uint8_t* srow;  // MXFP4: this lane's weight row's E8M0 scales
  const uint16_t* abase;              // x (up/gate) or mid (down)
  uint32_t act[max_tiles<NPRE>()];    // this lane's column per tile: activation offset + 32*lg
};

template <int NPRE>
__device__ inline void eat_job(const Params& p, const Lds& L, const Sched& s, Eat<NPRE>& e) {
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  const It& c = e.it;
  e.kc = 0;
  // consecutive jobs of one group (the down tiles of a CU's slice) share
  // the column lookups
  const int g = job_group(p, s, c), kind = c.phase <= 1 ? 1 : 2;
  const bool same = g == e.g && kind == e.kind;
  e.g = g;
  const bool sh = shared_group(p, e.g);
  e.kind = kind;
  e.fmt = sh ? 0 : p.routed_fmt;
  e.kdim = job_kdim(p, c, e.g);
  e.nck = nchunks(e.kdim);
  e.tile = job_tile(s, c);
  e.rt = c.phase == 2 ? c.rt : 0;
  e.nlive = e.kind == 2 ? (s.hc - 16 * e.rt < 16 ? s.hc - 16 * e.rt : 16) : 16;
  if (e.kind == 1) {
    e.split = 8;  // rows 0..7 of the MFMA tile are gate rows, 8..15 up rows
  } else {
    // a 16-row down tile spans at most two 128-row scale blocks
    const int hb = s.h0 + 16 * e.rt;
    e.split = (hb / 128 + 1) * 128 - hb;
  }
  int gstart = 0;
  if (same) {
  } else if (sh) {
    e.ncols = p.T;
  } else {
    uint32_t a, b, c;
    asm volatile("ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b), "=&v"(c)
                 : "v"(lds_off(L.gcnt + e.g)), "v"(lds_off(L.gstart + e.g)), "v"(lds_off(L.gexp + e.g))
                 : "memory");
    e.ncols = uni((int)a);
    gstart = uni((int)b);
    e.eid = uni((int)c);
  }
  const size_t eid = (size_t)e.eid;
  // the job's weight scales
  {
    const size_t H = p.H, I = p.I;
    const int iexp = sh ? p.Is : p.I;
    const int hb = s.h0 + 16 * e.rt;
    if (e.fmt == 0) {
      const float* S;
      if (sh) S = e.kind == 1 ? p.sh_sgu : p.sh_sd;
      else S = e.kind == 1 ? (const float*)p.sgu + eid * (2 * I / 128) * (H / 128)
                           : (const float*)p.sd + eid * (H / 128) * (I / 128);
      const int nkb = e.kdim / 128;
      const int nb_lo = e.kind == 1 ? (8 * e.tile) / 128 : hb / 128;
      const int nb_hi = e.kind == 1 ? (iexp + 8 * e.tile) / 128 : (hb + e.nlive - 1) / 128;
      const int kb = (lane & 31) * 8 + wave_id();
      e.sreg = (lane & 31) < e.nck && kb < nkb ? S[(size_t)(lane < 32 ? nb_lo : nb_hi) * nkb + kb] : 0.f;
    } else {
      const uint8_t* S = e.kind == 1 ? (const uint8_t*)p.sgu + eid * 2 * I * (H / 32)
                                     : (const uint8_t*)p.sd + eid * H * (I / 32);
      const int row = lane & 15;
      const int wr = e.kind == 1 ? (row < 8 ? 8 * e.tile + row : iexp + 8 * e.tile + row - 8)
                                 : hb + (row < e.nlive ? row : e.nlive - 1);
      e.srow = S + (size_t)wr * (e.kdim / 32);
    }
  }
  if (same) return;
  e.nct = (e.ncols + 15) >> 4;
  e.abase = e.kind == 1 ? p.x : p.mid;
  // a lane past the group's columns takes the last column: MFMA columns
  // are independent and that output is never stored
  int codes[max_tiles<NPRE>()];
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
    const int cc = ct * 16 + (lane & 15) < e.ncols ? ct * 16 + (lane & 15) : e.ncols - 1;
    codes[ct] = sh ? cc * 16 + p.K : gstart + cc;
  }
  if (!sh) {
    // the routed group's column codes, all tiles in one round trip
    if (max_tiles<NPRE>() == 1) {
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(codes[0]) : "v"(lds_off(L.cols + codes[0])) : "memory");
    } else {
      int c4[4];
      asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(c4[0]), "=&v"(c4[1]), "=&v"(c4[2]), "=&v"(c4[3])
                   : "v"(lds_off(L.cols + codes[0])), "v"(lds_off(L.cols + codes[max_tiles<NPRE>() > 1 ? 1 : 0])),
                     "v"(lds_off(L.cols + codes[max_tiles<NPRE>() > 2 ? 2 : 0])),
                     "v"(lds_off(L.cols + codes[max_tiles<NPRE>() > 3 ? 3 : 0]))
                   : "memory");
#pragma unroll
      for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) codes[ct] = c4[ct];
    }
  }
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
    const int code = codes[ct];
    e.act[ct] = (e.kind == 1 ? (uint32_t)(code >> 4) * (uint32_t)p.H
                             : ((uint32_t)(code >> 4) * (uint32_t)(p.K + 1) + (uint32_t)(code & 15)) *
                                   (uint32_t)p.mid_ld) +
                32u * lg;
  }
}

// Activations of column tile ct at K-block kb for this lane: the 8 bf16 at
// elements kb*128 + 32*(lane >> 4) + 8m .. +7 of its column's row (x for
// up/gate, the mid line for down).
template <int NPRE>
__device__ __forceinline__ void load_tile(const Eat<NPRE>& e, int kb, int ct, u32x4* B) {
  const uint16_t* ptr = e.abase + e.act[ct] + kb * 128;
#pragma unroll
  for (int m = 0; m < 4; ++m) B[m] = ld16(ptr + 8 * m);
}

// The activations of chunk e.kc for tiles 0..NPRE-1, one chunk ahead of
// their use.  Every register is loaded on every call (a wave past the
// chunk's K range loads the last block again): a register that is only
// sometimes loaded makes the compiler wait for all loads before the merge.
template <int NPRE>
__device__ inline void load_pre(const Eat<NPRE>& e, Pre<NPRE>& P) {
  const int nkb = (e.kdim + 127) >> 7;
  const int kb = e.kc * 8 + wave_id() < nkb ? e.kc * 8 + wave_id() : nkb - 1;
#pragma unroll
  for (int ct = 0; ct < NPRE; ++ct) load_tile(e, kb, ct, P.B + 4 * ct);
  if (e.fmt != 0) P.sw = *(const uint32_t*)(e.srow + 4 * kb);
}

// Marks every prefetched register as read here, on every path: the wait for
// them then happens once, at this point.
template <int NPRE>
__device__ __forceinline__ void settle_pre(const Pre<NPRE>& P, int fmt) {
#pragma unroll
  for (int i = 0; i < 4 * NPRE; ++i) asm volatile("" ::"v"(P.B[i]));
  if (fmt != 0) asm volatile("" ::"v"(P.sw));
}

// Multiplies this wave's K-block of the chunk in `stage` into acc[ct].
// FP8: a 4-MFMA block sum per K-block, then times its 128x128 block scale.
// MXFP4: the E8M0 scale is folded into the exact bf16 conversion.
// This wave's weights of a chunk, copied out of the stage so the stage can
// be released before the math: FP8 32 bytes per lane, MXFP4 16.
struct Raw {
  u32x4 a0, a1;
};

// False when the wave has no K-block in this chunk (a ragged last chunk).
template <int F, int NPRE>
__device__ __forceinline__ bool fetch_chunk(const Eat<NPRE>& e, const lds_char* stage, Raw& r) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const int wave = wave_id();
  if ((e.kc * 8 + wave) * 128 >= e.kdim) return false;
  if (F == 0) lds_ld_fp8_block(stage + row * kPitch + wave * 128 + 32 * lg, r.a0, r.a1);
  else lds_ld_fp4_block(stage + row * kPitch + wave * 64 + 16 * lg, r.a0);
  return true;
}

template <int F, int NPRE>
__device__ inline void compute_chunk(const Eat<NPRE>& e, const Raw& r, const Pre<NPRE>& P, f32x4* acc) {
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  const int kb = e.kc * 8 + wave_id();
  bf16x8 A[4];
  float s_lo = 1.f, s_hi = 1.f;
  if (F == 0) {
    A[0] = e4m3x8_to_bf16(r.a0[0], r.a0[1]);
    A[1] = e4m3x8_to_bf16(r.a0[2], r.a0[3]);
    A[2] = e4m3x8_to_bf16(r.a1[0], r.a1[1]);
    A[3] = e4m3x8_to_bf16(r.a1[2], r.a1[3]);
    s_lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e.sreg), e.kc));
    s_hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e.sreg), 32 + e.kc));
  } else {
    const float sc = e8m0_to_f32((P.sw >> (8 * lg)) & 0xffu);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(r.a0[m], sc);
  }
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
    if (ct < e.nct) {
      u32x4 Bl[4];
      const u32x4* B = P.B + 4 * (ct < NPRE ? ct : 0);
      if (ct >= NPRE) {
        load_tile(e, kb, ct, Bl);
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

// Job-end reductions.  At the end of a job every compute wave stores its
// partial tiles into partial slot (job % slots) and raises its part count;
// it never waits for the others there.  Job j is summed by its owner wave
// (j mod 8) later: at the owner's next job end, at the up/gate -> down
// hand-over, or while the owner waits for a slot.  The sum runs over the
// waves in order 0..7, exactly as a workgroup-wide reduction would.  A slot
// is reused for job j only after job j - slots was summed out of it.
template <int NPRE>
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

template <int NPRE>
__device__ __forceinline__ const float* red_slot(const Lds& L, int T, int jc) {
  return L.red + (size_t)(jc % red_slots(T)) * red_tiles(T) * (kRedTileBytes / 4);
}

// Sums the owned job out of its slot.  Lane l holds MFMA rows 4*(l>>4)+q of
// column (l & 15) in every wave's partial.  Up/gate: rows 0..7 are gate
// rows, 8..15 (32 lanes on) the matching up rows; lanes 0..31 each finish
// four intermediates, mid = silu(gate) * up rounded to bf16.  Down: every
// lane finishes its four rows into the LDS products.
template <int NPRE>
__device__ inline void sum_job(const Params& p, const Lds& L, const Owned<NPRE>& o) {
  const int lane = threadIdx.x & 63;
  const float* base = red_slot<NPRE>(L, p.T, o.jc);
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
              const float m = g / (1.0f + expf(-g)) * u;
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
            const size_t at = ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.hs + 16 * o.rt + i;
            if (NPRE == 1) lds_st32(L.pbuf + at, __float_as_uint(v));
            else p.prod[(size_t)blockIdx.x * p.T * (p.K + 1) * p.hs + at] = v;
          }
        }
      }
    }
  }
}

// Sums the owned job when every wave's partials are in (or waits for them
// when `block`), then releases its slot.
template <int NPRE>
__device__ inline void service(const Params& p, const Lds& L, Owned<NPRE>& o, bool block, bool& ok) {
  o.jc = uni(o.jc);
  if (o.jc < 0) return;
  if (block) lds_wait<8>(p, L.ctl + kCtlPart, (uint32_t)(o.jc + 1), ok);
  else if (ok && (int)lds_min<8>(L.ctl + kCtlPart) < o.jc + 1) return;
  sum_job(p, L, o);
  lds_st32(L.ctl + kCtlSlot + o.jc % red_slots(p.T), (uint32_t)(o.jc + 1));
  o.jc = -1;
}

// End of job jc for this wave: wait for its slot (summing an owned job
// meanwhile), store the partial tiles, raise the part count, finish an older
// owned job, and take ownership of jc when it is this wave's.
template <int NPRE>
__device__ inline void job_end(const Params& p, const Lds& L, const Eat<NPRE>& e, f32x4* acc, int jc,
                               Owned<NPRE>& own, bool& ok) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int ns = red_slots(p.T);
  if (jc >= ns) {
    const uint32_t target = (uint32_t)(jc - ns + 1);
    const uint32_t* sd = L.ctl + kCtlSlot + jc % ns;
    int spins = 0;
    while (ok && lds_min<1>(sd) < target) {
      service(p, L, own, false, ok);
      if (++spins > kSpinLimit) {
        set_err(p.err, kErrTimeout);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  float* base = (float*)red_slot<NPRE>(L, p.T, jc);
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct)
    if (ct < e.nct)
      lds_st128(base + (size_t)ct * (kRedTileBytes / 4) + ((size_t)wave * 64 + lane) * 4,
                __builtin_bit_cast(u32x4, acc[ct]));
  lds_st32(L.ctl + kCtlPart + wave, (uint32_t)(jc + 1));
  service(p, L, own, true, ok);
  if (jc % kWaves == wave) {
    own.jc = jc;
    own.kind = e.kind;
    own.g = e.g;
    own.tile = e.tile;
    own.rt = e.rt;
    own.ncols = e.ncols;
    own.nct = e.nct;
    own.nlive = e.nlive;
  }
#pragma unroll
  for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// out[r][h] = P_shared + sum_p w[r][p] * P[r][p], fp32 FMA chain in slot
// order, rounded to bf16 once.
// The products are in LDS for batches of at most 16 rows, else in this
// CU's part of the workspace.
template <int NPRE>
__device__ inline void combine(const Params& p, const Lds& L, const Sched& s) {
  const float* P = NPRE == 1 ? L.pbuf : p.prod + (size_t)blockIdx.x * p.T * (p.K + 1) * p.hs;
  for (int t = threadIdx.x; t < p.T * s.hc; t += kThreads) {
    const int r = t / s.hc, hl = t - r * s.hc;
    const float* pr = P + (size_t)r * (p.K + 1) * p.hs + hl;
    float acc = p.n_shared ? pr[(size_t)p.K * p.hs] : 0.f;
    for (int k = 0; k < p.K; ++k) acc = fmaf(L.w[r * p.K + k], pr[(size_t)k * p.hs], acc);
    p.out[(size_t)r * p.H + s.h0 + hl] = (uint16_t)f32_to_bf16_rne(acc);
  }
}

// ------------------------------------------------------------------ kernel

template <int MODE, int FMT, int NPRE>
__global__ __launch_bounds__(kThreads, 1) void moe_fused(Params p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Lds L = lds_map(smem, p);
  lds_char* const st3 = (lds_char*)(smem + (L.stages - smem));
  const int tid = threadIdx.x, wave = wave_id();
  const bool producer = wave >= kWaves;
  const int pw = wave - kWaves;

  MOE_STAMP(p, 0);
  if (tid < 64) L.ctl[tid] = 0u;
  if (tid == 0)
    L.misc[1] = (int32_t)__hip_atomic_load(&p.flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t epoch = (uint32_t)__builtin_amdgcn_readfirstlane(L.misc[1]);

  Sched s;
  s.sh_tiles = (MODE == kModeForward && p.n_shared) ? p.Is / 8 : 0;
  s.rt_tiles = p.I / 8;
  s.n_jobs = 0;
  s.G = 0;
  s.routed = 0;
  s.h0 = blockIdx.x * p.hs;
  s.hc = p.H - s.h0 < p.hs ? p.H - s.h0 : p.hs;
  if (s.hc < 0) s.hc = 0;
  s.nrt = (s.hc + 15) / 16;

  // Producer waves stream weight chunks into the LDS ring; they issue no
  // other vector memory operation, so their in-order vmcnt tracks the ring
  // exactly, and the compute waves' activation loads never queue behind a
  // DMA.
  Feed feed;
  feed.it = It{0, first_job(p, 0), 0, 0, 0};
  feed.kc = 0;
  int n_i = 0, n_c = 0;
  settle(p, s, feed.it);
  // S1: the shared expert's up/gate chunks need no routing: start them now
  if (MODE == kModeForward && producer) {
    __builtin_amdgcn_s_setprio(3);
    while (n_i < p.ns - 1 && feed.it.phase < 3 && !blocked(s, feed.it)) {
      if (feed.kc == 0) feed_job(p, L, s, feed, pw);
      feed_chunk(feed, st3 + (n_i % p.ns) * kStageBytes, pw);
      ++n_i;
      if (++feed.kc == feed.nck) {
        feed.kc = 0;
        next_job(p, s, feed.it);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // S0: router logits of this CU's experts, published for every CU
  router_logits(p);
  publish(p, epoch + 1);
  MOE_STAMP(p, 1);
  if (MODE != kModeForward && blockIdx.x != 0) return;

  // S2: route every row, then group the step's distinct experts
  wait_all(p, epoch + 1);
  MOE_STAMP(p, 2);
  if (!producer)
    for (int r = wave; r < p.T; r += kWaves) route_row(p, L, r);
  __syncthreads();
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
    // g differs per thread here, so plain LDS reads (no DMA is in flight)
    for (int g = tid; g < G; g += kThreads) {
      o[4 + g] = p.n_shared && g == 0 ? -1 : L.gexp[g];
      o[4 + G + g] = p.n_shared && g == 0 ? p.T : L.gcnt[g];
      o[4 + 2 * G + g] = p.n_shared && g == 0 ? 0 : L.gstart[g];
    }
    const int ncol = p.T * (p.K + p.n_shared);
    for (int c = tid; c < ncol; c += kThreads) o[4 + 3 * G + c] = L.cols[c];
    return;
  }
  s.G = G;
  s.n_jobs = s.sh_tiles + (G - p.n_shared) * s.rt_tiles;
  s.routed = 1;
  settle(p, s, feed.it);
  It start = It{0, first_job(p, 0), 0, 0, 0};
  settle(p, s, start);

  // S3 / S4: the chunk stream.  The second flag (every CU's mid is out) is
  // raised after this CU's last up/gate job and awaited before the first
  // down chunk's activations are read; only the compute waves take part.
#ifdef MOE_LAPS
  uint64_t cyc[6] = {0, 0, 0, 0, 0, 0};
  uint64_t tq = __builtin_amdgcn_s_memtime();
#define MOE_LAP(i)                                    \
  do {                                                \
    const uint64_t t2 = __builtin_amdgcn_s_memtime(); \
    cyc[i] += t2 - tq;                                \
    tq = t2;                                          \
  } while (0)
#else
#define MOE_LAP(i) \
  do {             \
  } while (0)
#endif
  bool ok = true;

  // The producers and the compute waves never meet at a workgroup barrier
  // inside the stream: they hand chunks over through LDS counters.  A
  // producer keeps up to ns - 1 chunks in flight; when the oldest has
  // landed (its in-order vmcnt says so) it raises its ready count, and it
  // refills a stage once every compute wave's done count has passed the
  // chunk that stage held.  A compute wave waits for both producers' ready
  // counts, multiplies the chunk, raises its done count, and prefetches the
  // next chunk's activations.  Per-job descriptors are computed when a job
  // starts; a chunk only moves offsets.
  if (producer) {
    // The producers are the workgroup's youngest waves; the SIMD arbiter
    // favours older waves, so without a raised priority the compute waves
    // sharing their SIMDs starve the DMA issue.
    __builtin_amdgcn_s_setprio(3);
    int n_r = 0;       // chunks this wave has reported landed
    uint32_t cdone = 0;  // last read minimum of the compute waves' done counts
    for (;;) {
      n_i = uni(n_i);
      n_r = uni(n_r);
      uni(feed.it);
      feed.kc = uni(feed.kc);
      if (feed.it.phase >= 3) break;
      if (feed.kc == 0) feed_job(p, L, s, feed, pw);
      // room for chunk n_i: fewer than ns - 1 chunks in flight, and its
      // stage released by every compute wave; meanwhile report landings
      while (n_i - n_r >= p.ns - 1 || (ok && n_i - (int)cdone >= p.ns)) {
        if (n_i - (int)cdone >= p.ns) cdone = lds_min<8>(L.ctl + kCtlDone);
        if (n_i - n_r >= p.ns - 1 || (n_r < n_i && n_i - (int)cdone >= p.ns)) {
          wait_vm(8 * (n_i - 1 - n_r));
          ++n_r;
          lds_st32(L.ctl + kCtlReady + pw, (uint32_t)n_r);
        } else if (n_i - (int)cdone >= p.ns) {
          lds_wait<8>(p, L.ctl + kCtlDone, (uint32_t)(n_i - p.ns + 1), ok);
          cdone = (uint32_t)(n_i - p.ns + 1);
        }
        n_r = uni(n_r);
      }
      MOE_LAP(0);
      feed_chunk(feed, st3 + (n_i % p.ns) * kStageBytes, pw);
      ++n_i;
      if (++feed.kc == feed.nck) {
        feed.kc = 0;
        next_job(p, s, feed.it);
      }
      MOE_LAP(1);
    }
    while (n_r < n_i) {
      wait_vm(8 * (n_i - 1 - n_r));
      ++n_r;
      lds_st32(L.ctl + kCtlReady + pw, (uint32_t)n_r);
    }
    n_c = n_r;
    __builtin_amdgcn_s_setprio(0);
  } else {
    constexpr int MAXCT = max_tiles<NPRE>();
    const int wave_c = wave;
    bool passed2 = false;
    // every compute wave has completed its mid stores; wave 0 publishes and,
    // when this CU has down work, waits for every CU and tells the others
    int jc = 0;  // jobs ended
    Owned<NPRE> own;
    own.jc = -1;
    auto cross_to_down = [&](const It& c) {
      if (!passed2 && c.phase >= 2) {
        MOE_STAMP(p, 4);
        service(p, L, own, true, ok);  // this wave's last owned up/gate job
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_st32(L.ctl + kCtlMidOut + wave_c, 1u);
        if (wave_c == 0) {
          lds_wait<8>(p, L.ctl + kCtlMidOut, 1u, ok);
          if (threadIdx.x == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_store(&p.flags[blockIdx.x], epoch + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if (c.phase == 2) poll_flags(p, epoch + 2);
          lds_st32(L.ctl + kCtlCrossed, 1u);
        }
        if (c.phase == 2) lds_wait<1>(p, L.ctl + kCtlCrossed, 1u, ok);
        MOE_STAMP(p, 5);
        passed2 = true;
      }
    };
    Eat<NPRE> e;
    e.it = start;
    e.g = -1;
    e.kind = 0;
    e.eid = 0;
    Pre<NPRE> pre;
    f32x4 acc[MAXCT];
#pragma unroll
    for (int ct = 0; ct < MAXCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t rdy = 0;  // last seen minimum of the producers' ready counts
    cross_to_down(e.it);
    if (e.it.phase < 3) {
      eat_job(p, L, s, e);
      load_pre(e, pre);
    }
    while (e.it.phase < 3) {
      n_c = uni(n_c);
      rdy = (uint32_t)uni((int)rdy);
      uni(e.it);
      e.kc = uni(e.kc);
      e.nck = uni(e.nck);
      e.nct = uni(e.nct);
      e.kind = uni(e.kind);
      e.fmt = uni(e.fmt);
      MOE_LAP(0);
      if ((int)rdy <= n_c) rdy = lds_wait<2>(p, L.ctl + kCtlReady, (uint32_t)(n_c + 1), ok);
      MOE_LAP(1);
      const lds_char* stage = st3 + (n_c % p.ns) * kStageBytes;
      Raw raw;
      const bool live = e.fmt == 0 ? fetch_chunk<0>(e, stage, raw) : fetch_chunk<FMT>(e, stage, raw);
      lds_st32(L.ctl + kCtlDone + wave, (uint32_t)(n_c + 1));  // the stage is free for this wave
      settle_pre(pre, e.fmt);
      if (live) {
        if (e.fmt == 0) compute_chunk<0>(e, raw, pre, acc);
        else compute_chunk<FMT>(e, raw, pre, acc);
      }
      MOE_LAP(2);
      if (e.kc == e.nck - 1) job_end(p, L, e, acc, jc++, own, ok);
      MOE_LAP(3);
      ++n_c;
      if (++e.kc == e.nck) {
        next_job(p, s, e.it);
        cross_to_down(e.it);
        MOE_LAP(4);
        if (e.it.phase < 3) eat_job(p, L, s, e);
        MOE_LAP(0);
      }
      MOE_LAP(4);
      if (e.it.phase >= 3) break;
      load_pre(e, pre);
      MOE_LAP(5);
    }
    service(p, L, own, true, ok);  // the last owned down job
  }
#ifdef MOE_LAPS
  if (p.timeline && (threadIdx.x == 0 || threadIdx.x == 64 * kWaves)) {
    if (threadIdx.x == 0)
      for (int i = 0; i < 6; ++i) p.timeline[blockIdx.x * 16 + 10 + i] = cyc[i];
    else
      for (int i = 0; i < 6; ++i) p.timeline[1024 * 16 - 256 * 8 + blockIdx.x * 8 + i] = cyc[i];
  }
#endif
  MOE_STAMP(p, 6);
  __syncthreads();

  // S5: combine this CU's output rows
  combine<NPRE>(p, L, s);
  MOE_STAMP(p, 7);
  if (threadIdx.x == 0 && p.timeline) {
    p.timeline[blockIdx.x * 16 + 8] = (uint64_t)n_c;
    p.timeline[blockIdx.x * 16 + 9] = (uint64_t)p.ns;
  }
}

// ------------------------------------------------------------------ host glue

WsLayout ws_layout(int max_rows, int E, int K, int H, int I, int Is) {
  WsLayout w;
  size_t q = 0;
  w.flags = q; q = align_up(q + 4 * 1024, 256);
  w.err = q; q = align_up(q + 256, 256);
  w.scores = q; q = align_up(q + 16 * (size_t)max_rows * E, 256);
  w.mid_ld = (I > Is ? I : Is);
  w.mid = q; q = align_up(q + 2 * (size_t)max_rows * (K + 1) * w.mid_ld, 256);
  // ncu * hs <= H + ncu - 1 and ncu <= 1024, so H + 1024 rows of products cover every CU's slice
  w.prod = q;
  if (max_rows > kLdsProdRows) q = align_up(q + 4 * (size_t)max_rows * (K + 1) * (H + 1024), 256);
  w.total = q;
  return w;
}

template <int MODE, int FMT, int NPRE = 1>
static hipError_t launch_one(const Params& p, hipStream_t stream) {
  auto kfn = moe_fused<MODE, FMT, NPRE>;
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(p.ncu), dim3(kThreads), p.lds_bytes, stream, p);
  return hipGetLastError();
}

hipError_t launch(const Params& p, int mode, hipStream_t stream) {
  const bool wide = p.T > 16;  // some group may have more than one 16-column tile
  if (p.routed_fmt == 0) {
    if (mode == kModeForward)
      return wide ? launch_one<kModeForward, 0, 2>(p, stream) : launch_one<kModeForward, 0, 1>(p, stream);
    if (mode == kModeRoute) return launch_one<kModeRoute, 0>(p, stream);
    return launch_one<kModeGroups, 0>(p, stream);
  }
  if (mode == kModeForward)
    return wide ? launch_one<kModeForward, 1, 2>(p, stream) : launch_one<kModeForward, 1, 1>(p, stream);
  if (mode == kModeRoute) return launch_one<kModeRoute, 1>(p, stream);
  return launch_one<kModeGroups, 1>(p, stream);
}

}  // namespace moe
