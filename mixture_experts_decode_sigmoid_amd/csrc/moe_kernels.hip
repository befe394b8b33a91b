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
constexpr int kScaleOff = 16 * kPitch;          // the chunk's weight scales follow its rows
constexpr int kStageBytes = kScaleOff + 512;
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
  float* red;        // [kWaves][64][4] cross-wave reduction
  double* rb;        // [kWaves][E] router keys (aliases pbuf)
  double* rgs;       // [kWaves][64] group scores
  int32_t* rkept;    // [kWaves][64]
  float* pbuf;       // [T*(K+1)][hs] down products
  char* stages;      // [ns][kStageBytes]
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct LdsOffsets {
  size_t ids, w, first, egrp, rmask, gexp, gcnt, gstart, cols, misc, red, pbuf, stages;
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
  o.red = q; q = align_up(q + 16 * (size_t)kWaves * 64, 16);
  o.pbuf = q;
  size_t pb = 4 * (size_t)T * (K + 1) * hs;
  size_t rs = 8 * (size_t)kWaves * E + 8 * (size_t)kWaves * 64 + 4 * (size_t)kWaves * 64;
  q = align_up(q + (pb > rs ? pb : rs), 16);
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
  L.red = (float*)(base + o.red);
  L.pbuf = (float*)(base + o.pbuf);
  L.rb = (double*)(base + o.pbuf);
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
__device__ inline void wait_all(const Params& p, uint32_t target) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
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
// order, then a fixed xor butterfly; one wave per (row, expert).
__device__ inline void router_logits(const Params& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= kWaves) return;
  for (int e = blockIdx.x; e < p.E; e += p.ncu) {
    const uint16_t* wr = p.router_w + (size_t)e * p.H;
    const double bias = load_bias(p, e);
    for (int r = wave; r < p.T; r += kWaves) {
      const uint16_t* xr = p.x + (size_t)r * p.H;
      double acc = 0.0;
      for (int h = 8 * lane; h < p.H; h += 512) {
        u32x4 xv = ld16(xr + h), wv = ld16(wr + h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t xa = xv[j], wa = wv[j];
          acc = fma((double)bf16_bits_to_f32(xa & 0xffffu), (double)bf16_bits_to_f32(wa & 0xffffu), acc);
          acc = fma((double)bf16_bits_to_f32(xa >> 16), (double)bf16_bits_to_f32(wa >> 16), acc);
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
  double bv[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    alive[i] = e < p.E;
    double b = alive[i] ? sc[2 * e + 1] : -INFINITY;
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
      picks[k] = be;
      ssum += sc[2 * be];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (k < p.K) {
        const int e = picks[k];
        L.ids[r * p.K + k] = e;
        L.w[r * p.K + k] = (float)(sc[2 * e] / ssum * p.routed_scale);
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
// outstanding (n is a multiple of 9: a producer issues 9 DMAs per chunk).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
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
__device__ __forceinline__ void lds_st32(void* p, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st128(void* p, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_off(p)), "v"(v) : "memory");
}
// A lane's part of one K-block of the stage with its scales, in one round
// trip: FP8, 32 weight bytes and the two 128-row block scales (the second
// one 32 bytes after the first); MXFP4, 16 weight bytes and a dword of the
// row's E8M0 scales.
template <class P>
__device__ __forceinline__ void lds_ld_fp8_block(P w, P sc, u32x4& a, u32x4& b, uint32_t& s0, uint32_t& s1) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b32 %2, %5\n\tds_read_b32 %3, %5 offset:32\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(s0), "=&v"(s1)
      : "v"(lds_off(w)), "v"(lds_off(sc))
      : "memory");
}
template <class P>
__device__ __forceinline__ void lds_ld_fp4_block(P w, P sc, u32x4& a, uint32_t& s0) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(s0)
               : "v"(lds_off(w)), "v"(lds_off(sc))
               : "memory");
}

// Per-lane prefetch of one chunk: the activations of column tiles
// 0..NPRE-1 (later tiles are loaded when used), and where the FP8 scale
// changes inside the 16-row weight tile.  NPRE is 1 for batches of at most
// 16 rows (no group has more than 16 columns) and 2 above.
template <int NPRE>
struct Pre {
  u32x4 B[4 * NPRE];
  int split;         // FP8: MFMA output rows (4*lg + q) below it take the first scale
  int nct;
};

// Column tiles a group can have: 1 when NPRE is 1, else up to 4 (64 rows).
template <int NPRE>
constexpr int max_tiles() { return NPRE == 1 ? 1 : kMaxRows / 16; }

struct Pos {
  int phase;  // 0 shared up/gate, 1 routed up/gate, 2 down, 3 end
  int j;      // up/gate: global job index; down: group
  int rt;     // down: 16-row tile of this CU's slice
  int kc;     // chunk along the reduction axis
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

struct Chunk {
  int kind;  // 1 up/gate, 2 down
  int g, tile, rt, kc;
  int fmt, iexp, kdim, nlive;
  const uint8_t* w;
  const void* s;
};

__device__ __forceinline__ int nchunks(int kdim) { return (kdim + kChunkElems - 1) / kChunkElems; }

// Smallest j >= begin with j = blockIdx.x (mod ncu): jobs are dealt round-robin.
__device__ __forceinline__ int first_job(const Params& p, int begin) {
  const int r = begin % p.ncu;
  return begin + (((int)blockIdx.x - r) % p.ncu + p.ncu) % p.ncu;
}

__device__ __forceinline__ int chunk_count(const Params& p, const Pos& c) {
  if (c.phase <= 1) return nchunks(p.H);
  return nchunks((p.n_shared && c.j == 0) ? p.Is : p.I);
}

__device__ __forceinline__ bool blocked(const Sched& s, const Pos& c) {
  return c.phase == 0 && c.j >= s.sh_tiles;  // routed work before routing is known
}

__device__ inline void settle(const Params& p, const Sched& s, Pos& c) {
  for (;;) {
    if (c.phase == 0) {
      if (c.j < s.sh_tiles || !s.routed) return;
      c.phase = 1;
      c.j = first_job(p, s.sh_tiles);
      c.kc = 0;
      continue;
    }
    if (c.phase == 1) {
      if (c.j < s.n_jobs) return;
      c.phase = 2;
      c.j = 0;
      c.rt = 0;
      c.kc = 0;
      continue;
    }
    if (c.phase == 2 && (s.nrt <= 0 || c.j >= s.G)) c.phase = 3;
    return;
  }
}

__device__ inline void advance(const Params& p, const Sched& s, Pos& c) {
  if (++c.kc < chunk_count(p, c)) return;
  c.kc = 0;
  if (c.phase <= 1) {
    c.j += p.ncu;
  } else if (++c.rt >= s.nrt) {
    c.rt = 0;
    ++c.j;
  }
  settle(p, s, c);
}

// Weights of group g: the shared expert (group 0 when present) or routed
// expert gexp[g].
__device__ inline void group_weights(const Params& p, const Lds& L, int g, Chunk& k, bool down) {
  if (p.n_shared && g == 0) {
    k.fmt = 0;
    k.iexp = p.Is;
    k.w = down ? p.sh_wd : p.sh_wgu;
    k.s = down ? (const void*)p.sh_sd : (const void*)p.sh_sgu;
    return;
  }
  const size_t e = (size_t)lds_ldi_uniform(L.gexp + g);
  const size_t H = p.H, I = p.I;
  k.fmt = p.routed_fmt;
  k.iexp = p.I;
  if (p.routed_fmt == 0) {
    // W_gate_up [E][2I][H], W_down [E][H][I] bytes; fp32 scales per 128x128
    if (down) {
      k.w = p.wd + e * H * I;
      k.s = (const float*)p.sd + e * (H / 128) * (I / 128);
    } else {
      k.w = p.wgu + e * 2 * I * H;
      k.s = (const float*)p.sgu + e * (2 * I / 128) * (H / 128);
    }
  } else {
    // W_gate_up [E][2I][H/2], W_down [E][H][I/2] bytes; E8M0 per 32 along K
    if (down) {
      k.w = p.wd + e * H * (I / 2);
      k.s = (const uint8_t*)p.sd + e * H * (I / 32);
    } else {
      k.w = p.wgu + e * 2 * I * (H / 2);
      k.s = (const uint8_t*)p.sgu + e * 2 * I * (H / 32);
    }
  }
}

// Group of an up/gate position: the shared expert's jobs come first, then
// rt_tiles jobs per routed group.
__device__ __forceinline__ int chunk_group(const Params& p, const Sched& s, const Pos& c) {
  return c.phase == 0 ? 0 : p.n_shared + (c.j - s.sh_tiles) / s.rt_tiles;
}

__device__ inline Chunk chunk_of(const Params& p, const Lds& L, const Sched& s, const Pos& c) {
  Chunk k;
  k.kc = c.kc;
  if (c.phase <= 1) {
    k.kind = 1;
    k.g = chunk_group(p, s, c);
    k.tile = c.phase == 0 ? c.j : (c.j - s.sh_tiles) % s.rt_tiles;
    k.rt = 0;
    group_weights(p, L, k.g, k, false);
    k.kdim = p.H;
    k.nlive = 16;
  } else {
    k.kind = 2;
    k.g = c.j;
    k.tile = 0;
    k.rt = c.rt;
    group_weights(p, L, k.g, k, true);
    k.kdim = k.iexp;
    k.nlive = s.hc - 16 * c.rt < 16 ? s.hc - 16 * c.rt : 16;
  }
  return k;
}

// Weight row n of chunk row r: up/gate rows 0..7 are gate rows 8t..8t+7 and
// rows 8..15 the up rows I+8t..I+8t+7; down rows are output rows h0+16rt+r.
__device__ __forceinline__ int weight_row_index(const Sched& s, const Chunk& k, int r) {
  if (k.kind == 1) return r < 8 ? 8 * k.tile + r : k.iexp + 8 * k.tile + r - 8;
  return s.h0 + 16 * k.rt + r;
}

// Producer wave pw streams rows 8pw..8pw+7 of a chunk (8 DMA instructions,
// always issued: a row past the live rows has no valid bytes) and one DMA of
// scales, so its vmcnt bookkeeping is 9 per chunk.  Scales land at
// kScaleOff: FP8, 16 floats from producer 0 (the 8 K-blocks' scales of the
// tile's first and second 128-row block); MXFP4, 32 E8M0 bytes per row.
__device__ inline void issue_chunk(const Params& p, const Lds& L, const Sched& s, const Pos& c,
                                   lds_char* stage, int pw) {
  const Chunk k = chunk_of(p, L, s, c);
  const int lane = threadIdx.x & 63;
  const int cbytes = k.fmt ? kChunkElems / 2 : kChunkElems;
  const int rowbytes = __builtin_amdgcn_readfirstlane(k.fmt ? k.kdim / 2 : k.kdim);
  const int koff = k.kc * cbytes;
  const int left = rowbytes - koff;
  const int nbytes = __builtin_amdgcn_readfirstlane(left < cbytes ? left : cbytes);
  // this wave's 8 chunk rows are consecutive weight rows (gate rows, up
  // rows, or output rows), so one base and the row pitch address them all
  const int nl = __builtin_amdgcn_readfirstlane(k.nlive - 8 * pw);
  const uint8_t* b = (const uint8_t*)uniform_ptr(
      k.w + (size_t)weight_row_index(s, k, nl > 0 ? 8 * pw : 0) * rowbytes + koff);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    dma_row(q < nl ? b + q * rowbytes : b, q < nl ? nbytes : 0, stage + (8 * pw + q) * kPitch);
  const uint32_t kOob = 0x7ffffff0u;
  uint32_t voff = kOob, nrec;
  if (k.fmt == 0) {
    const int nkb = k.kdim / 128;
    int nb_lo, nb_hi, nrows;
    if (k.kind == 1) {
      nb_lo = (8 * k.tile) / 128;
      nb_hi = (k.iexp + 8 * k.tile) / 128;
      nrows = 2 * k.iexp / 128;
    } else {
      const int hb = s.h0 + 16 * k.rt;
      nb_lo = hb / 128;
      nb_hi = (hb + k.nlive - 1) / 128;
      nrows = p.H / 128;
    }
    const int kb = k.kc * 8 + (lane & 7);
    if (pw == 0 && lane < 16 && kb < nkb) voff = (uint32_t)(((lane < 8 ? nb_lo : nb_hi) * nkb + kb) * 4);
    nrec = (uint32_t)(nrows * nkb * 4);
  } else {
    const int spr = k.kdim / 32;                 // scale bytes per weight row
    const int r = 8 * pw + (lane >> 3), d = lane & 7;
    const int valid = spr - k.kc * 32 < 32 ? spr - k.kc * 32 : 32;
    if (r < k.nlive && 4 * d < valid) voff = (uint32_t)(weight_row_index(s, k, r) * spr + k.kc * 32 + 4 * d);
    nrec = (uint32_t)((k.kind == 1 ? 2 * k.iexp : p.H) * spr);
  }
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(k.s), 0,
                                                                __builtin_amdgcn_readfirstlane((int)nrec), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + kScaleOff + 256 * pw),
                                           4, voff, 0, 0, 0);
}

// Column c of group g as row*16 + slot.
__device__ __forceinline__ int col_code(const Params& p, const Lds& L, int g, int c) {
  if (p.n_shared && g == 0) return c * 16 + p.K;
  return (int)lds_ld32(L.cols + lds_ldi_uniform(L.gstart + g) + c);
}

__device__ __forceinline__ int group_ncols(const Params& p, const Lds& L, int g) {
  if (p.n_shared && g == 0) return p.T;
  return lds_ldi_uniform(L.gcnt + g);
}

// Activations of column tile ct at K-block kb for this lane: B[m] holds the
// 8 bf16 of column ct*16 + (lane & 15) at elements kb*128 + 32*(lane >> 4) +
// 8m .. +7 (x rows for up/gate, mid lines for down).  A lane past the
// group's columns loads the last column again: MFMA columns are independent
// and that output is never stored.
__device__ __forceinline__ void load_tile(const Params& p, const Lds& L, const Chunk& k, int kb,
                                          int ct, int ncols, u32x4* B) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const int c = ct * 16 + row < ncols ? ct * 16 + row : ncols - 1;
  const int code = col_code(p, L, k.g, c);
  const uint16_t* src = k.kind == 1
      ? p.x + (size_t)(code >> 4) * p.H
      : p.mid + ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.mid_ld;
  const uint16_t* ptr = src + kb * 128 + 32 * lg;
#pragma unroll
  for (int m = 0; m < 4; ++m) B[m] = ld16(ptr + 8 * m);
}

// Activations of the next chunk for this lane: for each 16-column tile
// ct < NPRE, B[4ct+m] holds the 8 bf16 of column ct*16 + (lane & 15) at
// elements kb*128 + 32*(lane >> 4) + 8m .. +7 (x rows for up/gate, mid lines
// for down), one chunk ahead of their use.  Every register is loaded on
// every call (a wave past the chunk's K range loads the last block again, a
// tile past the group's columns its last column): a register that is only
// sometimes loaded makes the compiler wait for all loads before the merge.
template <int NPRE>
__device__ inline void load_pre(const Params& p, const Lds& L, const Sched& s, const Chunk& k, Pre<NPRE>& P) {
  const int nkb = (k.kdim + 127) >> 7;
  const int kb = k.kc * 8 + wave_id() < nkb ? k.kc * 8 + wave_id() : nkb - 1;
  const int ncols = group_ncols(p, L, k.g);
  P.nct = (ncols + 15) >> 4;
#pragma unroll
  for (int ct = 0; ct < NPRE; ++ct) load_tile(p, L, k, kb, ct, ncols, P.B + 4 * ct);
  if (k.kind == 1) {
    P.split = 8;  // rows 0..7 of the MFMA tile are gate rows, 8..15 up rows
  } else {
    // a 16-row down tile spans at most two 128-row scale blocks
    const int hb = s.h0 + 16 * k.rt;
    P.split = (hb / 128 + 1) * 128 - hb;
  }
}

// Multiplies this wave's K-block of the chunk in `stage` into acc[ct].
// FP8: a 4-MFMA block sum per K-block, then times its 128x128 block scale.
// MXFP4: the E8M0 scale is folded into the exact bf16 conversion.
// Marks every prefetched register as read here, on every path: the wait for
// them then happens once, at this point (vmcnt(2) in the steady state), and
// none of them is left with a load in flight that a later reuse of the
// register would have to wait out with vmcnt(0).
template <int NPRE>
__device__ __forceinline__ void settle_pre(const Pre<NPRE>& P) {
#pragma unroll
  for (int i = 0; i < 4 * NPRE; ++i) asm volatile("" ::"v"(P.B[i]));
}

template <int F, int NPRE>
__device__ inline void compute_chunk(const Params& p, const Lds& L, const Chunk& k,
                                     const lds_char* stage, const Pre<NPRE>& P, f32x4* acc) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, row = lane & 15;
  const int wave = wave_id();
  const int kb = k.kc * 8 + wave;
  if (kb * 128 >= k.kdim) return;
  bf16x8 A[4];
  if (F == 0) {
    u32x4 a0, a1;
    uint32_t slo, shi;
    lds_ld_fp8_block(stage + row * kPitch + wave * 128 + 32 * lg, stage + kScaleOff + 4 * wave, a0, a1, slo, shi);
    A[0] = e4m3x8_to_bf16(a0[0], a0[1]);
    A[1] = e4m3x8_to_bf16(a0[2], a0[3]);
    A[2] = e4m3x8_to_bf16(a1[0], a1[1]);
    A[3] = e4m3x8_to_bf16(a1[2], a1[3]);
    const float s_lo = __uint_as_float(slo), s_hi = __uint_as_float(shi);
#pragma unroll
    for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
      if (ct < P.nct) {
        u32x4 Bl[4];
        const u32x4* B = P.B + 4 * (ct < NPRE ? ct : 0);
        if (ct >= NPRE) {
          load_tile(p, L, k, kb, ct, group_ncols(p, L, k.g), Bl);
          B = Bl;
        }
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) t = mfma16(A[m], __builtin_bit_cast(bf16x8, B[m]), t);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ct][q] = fmaf(t[q], 4 * lg + q < P.split ? s_lo : s_hi, acc[ct][q]);
      }
    }
  } else {
    u32x4 a;
    uint32_t sw;
    lds_ld_fp4_block(stage + row * kPitch + wave * 64 + 16 * lg, stage + kScaleOff + row * 32 + 4 * wave, a, sw);
    const float sc = e8m0_to_f32((sw >> (8 * lg)) & 0xffu);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[m] = e2m1x8_to_bf16(a[m], sc);
#pragma unroll
    for (int ct = 0; ct < max_tiles<NPRE>(); ++ct) {
      if (ct < P.nct) {
        u32x4 Bl[4];
        const u32x4* B = P.B + 4 * (ct < NPRE ? ct : 0);
        if (ct >= NPRE) {
          load_tile(p, L, k, kb, ct, group_ncols(p, L, k.g), Bl);
          B = Bl;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[ct] = mfma16(A[m], __builtin_bit_cast(bf16x8, B[m]), acc[ct]);
      }
    }
  }
}

// End of an up/gate job: sum the 8 waves' K-block partials in wave order,
// mid = silu(gate) * up, rounded to bf16, stored at the column's (row, slot).
// Two workgroup barriers per column tile (the producer waves replay them).
template <int MAXCT>
__device__ inline void reduce_up(const Params& p, const Lds& L, const Chunk& k, f32x4* acc, int nct) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncols = group_ncols(p, L, k.g);
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) {
    if (ct < nct) {
      if (wave < kWaves) lds_st128(L.red + ((size_t)wave * 64 + lane) * 4, __builtin_bit_cast(u32x4, acc[ct]));
      bar_lds();
      if (tid < 128) {
        const int i = tid >> 4, cc = tid & 15, col = ct * 16 + cc;
        const int gl = (i >> 2) * 16 + cc, ul = gl + 32, q = i & 3;
        float g = 0.f, u = 0.f;
        for (int w = 0; w < kWaves; ++w) {
          g += lds_ldf(L.red + ((size_t)w * 64 + gl) * 4 + q);
          u += lds_ldf(L.red + ((size_t)w * 64 + ul) * 4 + q);
        }
        if (col < ncols) {
          const float m = g / (1.0f + expf(-g)) * u;
          if (!isfinite(m)) set_err(p.err, kErrMid);
          const int code = col_code(p, L, k.g, col);
          p.mid[((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.mid_ld + 8 * k.tile + i] =
              (uint16_t)f32_to_bf16_rne(m);
        }
      }
      bar_lds();
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// End of a down row tile: sum the waves' partials in wave order into the
// LDS products P[row][slot][h].
template <int MAXCT>
__device__ inline void reduce_down(const Params& p, const Lds& L, const Chunk& k, f32x4* acc, int nct) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncols = group_ncols(p, L, k.g);
#pragma unroll
  for (int ct = 0; ct < MAXCT; ++ct) {
    if (ct < nct) {
      if (wave < kWaves) lds_st128(L.red + ((size_t)wave * 64 + lane) * 4, __builtin_bit_cast(u32x4, acc[ct]));
      bar_lds();
      if (tid < 256) {
        const int ln = tid >> 2, q = tid & 3;
        const int i = 4 * (ln >> 4) + q, col = ct * 16 + (ln & 15);
        if (i < k.nlive && col < ncols) {
          float v = 0.f;
          for (int w = 0; w < kWaves; ++w) v += lds_ldf(L.red + ((size_t)w * 64 + ln) * 4 + q);
          if (!isfinite(v)) set_err(p.err, kErrMid);
          const int code = col_code(p, L, k.g, col);
          lds_st32(L.pbuf + ((size_t)(code >> 4) * (p.K + 1) + (code & 15)) * p.hs + 16 * k.rt + i,
                   __float_as_uint(v));
        }
      }
      bar_lds();
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// out[r][h] = P_shared + sum_p w[r][p] * P[r][p], fp32 FMA chain in slot
// order, rounded to bf16 once.
__device__ inline void combine(const Params& p, const Lds& L, const Sched& s) {
  for (int t = threadIdx.x; t < p.T * s.hc; t += kThreads) {
    const int r = t / s.hc, hl = t - r * s.hc;
    const float* pr = L.pbuf + (size_t)r * (p.K + 1) * p.hs + hl;
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
  Pos ipos = {0, first_job(p, 0), 0, 0}, cpos;
  int n_i = 0, n_c = 0;
  settle(p, s, ipos);
  // S1: the shared expert's up/gate chunks need no routing: start them now
  if (MODE == kModeForward && producer) {
    while (n_i < p.ns - 1 && ipos.phase == 0 && !blocked(s, ipos)) {
      issue_chunk(p, L, s, ipos, st3 + (n_i % p.ns) * kStageBytes, pw);
      advance(p, s, ipos);
      ++n_i;
    }
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
  settle(p, s, ipos);
  cpos = {0, first_job(p, 0), 0, 0};
  settle(p, s, cpos);

  // S3 / S4: the chunk stream.  The second flag (every CU's mid is out) is
  // raised after this CU's last up/gate job and awaited before the first
  // down chunk's activations are read.
  bool passed2 = false;
  auto cross_to_down = [&](const Pos& c) {
    if (!passed2 && c.phase >= 2) {
      MOE_STAMP(p, 4);
      publish(p, epoch + 2);
      if (c.phase == 2) wait_all(p, epoch + 2);
      MOE_STAMP(p, 5);
      passed2 = true;
    }
  };
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

  // One step: the producers wait for chunk n to land (the chunks after it
  // stay in flight), everyone meets, the compute waves multiply chunk n and
  // prefetch the activations of chunk n+1, a job ending here is reduced, and
  // the producers refill the stage chunk n-1 freed with chunk n+ns-1.
  // Producer and compute waves run separate loops that meet at the same
  // sequence of barriers: the top of each step, two per column tile of a
  // reduction, and the flag hand-over.  Kept apart, the producers' code
  // holds no load into a register, so nothing makes them drain the ring.
  if (producer) {
    while (ipos.phase < 3 && n_i < n_c + p.ns - 1) {
      issue_chunk(p, L, s, ipos, st3 + (n_i % p.ns) * kStageBytes, pw);
      advance(p, s, ipos);
      ++n_i;
    }
    cross_to_down(cpos);
    while (cpos.phase < 3) {
      wait_vm(9 * (n_i - 1 - n_c));
      MOE_LAP(0);
      bar_lds();
      MOE_LAP(1);
      if (cpos.kc == chunk_count(p, cpos) - 1) {
        const int g = cpos.phase <= 1 ? chunk_group(p, s, cpos) : cpos.j;
        const int nct = (group_ncols(p, L, g) + 15) >> 4;
        for (int ct = 0; ct < nct; ++ct) {
          bar_lds();
          bar_lds();
        }
      }
      MOE_LAP(3);
      advance(p, s, cpos);
      ++n_c;
      cross_to_down(cpos);
      MOE_LAP(4);
      if (ipos.phase < 3 && n_i < n_c + p.ns - 1) {
        issue_chunk(p, L, s, ipos, st3 + (n_i % p.ns) * kStageBytes, pw);
        advance(p, s, ipos);
        ++n_i;
      }
      MOE_LAP(5);
    }
  } else {
    constexpr int MAXCT = max_tiles<NPRE>();
    Pre<NPRE> pre;
    f32x4 acc[MAXCT];
#pragma unroll
    for (int ct = 0; ct < MAXCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    cross_to_down(cpos);
    if (cpos.phase < 3) load_pre(p, L, s, chunk_of(p, L, s, cpos), pre);
    while (cpos.phase < 3) {
      MOE_LAP(0);
      bar_lds();
      MOE_LAP(1);
      const Chunk k = chunk_of(p, L, s, cpos);
      const lds_char* stage = st3 + (n_c % p.ns) * kStageBytes;
      settle_pre(pre);
      if (k.fmt == 0) compute_chunk<0>(p, L, k, stage, pre, acc);
      else compute_chunk<FMT>(p, L, k, stage, pre, acc);
      MOE_LAP(2);
      if (cpos.kc == chunk_count(p, cpos) - 1) {
        if (k.kind == 1) reduce_up<MAXCT>(p, L, k, acc, pre.nct);
        else reduce_down<MAXCT>(p, L, k, acc, pre.nct);
      }
      MOE_LAP(3);
      advance(p, s, cpos);
      ++n_c;
      cross_to_down(cpos);
      MOE_LAP(4);
      if (cpos.phase >= 3) break;
      load_pre(p, L, s, chunk_of(p, L, s, cpos), pre);
      MOE_LAP(5);
    }
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
  if (!passed2) {
    publish(p, epoch + 2);
    passed2 = true;
  }
  __syncthreads();

  // S5: combine this CU's output rows
  combine(p, L, s);
  MOE_STAMP(p, 7);
  if (threadIdx.x == 0 && p.timeline) {
    p.timeline[blockIdx.x * 16 + 8] = (uint64_t)n_c;
    p.timeline[blockIdx.x * 16 + 9] = (uint64_t)p.ns;
  }
}

// ------------------------------------------------------------------ host glue

WsLayout ws_layout(int max_rows, int E, int K, int I, int Is) {
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
