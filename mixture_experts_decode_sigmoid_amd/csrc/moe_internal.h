// moe_internal.h -- parameter block shared by the host API (moe_api.cpp) and
// the device code (moe_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWaves = 8;                 // waves per workgroup (one workgroup per CU)
constexpr int kAllWaves = kWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxRows = 64;              // rows per call
constexpr int kMaxExperts = 256;          // routed experts (4 per lane in the router)
constexpr int kMaxTopK = 8;
constexpr int kMaxGroups = 64;            // router groups
constexpr int kMaxSlice = 64;             // output rows per CU in down
constexpr int kMinLds = 84 * 1024;        // LDS per workgroup: more than half a CU's, so one per CU

enum Mode {
  kModeForward = 0,
  kModeRoute = 1,
  kModeGroups = 2,
  // the unfused layout's shared-expert launches: gate/up only (mid to the
  // workspace), down only (from the workspace's mid to out, bf16)
  kModeSharedUp = 3,
  kModeSharedDown = 4,
};

// Activation loads per weight item (AL) by batch size: a job takes at most
// 4 * AL columns (a group with more columns is split into column tiles, each
// a job of its own), and every item of a kernel issues the same loads.
// Measured on the DeepSeek-V3 layer at 12 and 16 rows (and the MXFP4 layer
// at 16): two loads beat four by 12-16% and one by 5-7%.
__host__ __device__ inline int stream_al(int T) { return T <= 4 ? 1 : 2; }
// Down jobs are split over waves by K-phase up to this many rows; above it
// every wave claims whole down jobs (the K-phase partials would not fit LDS).
constexpr int kKsplitRows = 16;
// Intermediates per up/gate tile (ti).  An item is one 16-row MFMA tile (8
// gate rows and their 8 up rows), except with two activation loads per item
// in a kernel with MXFP4 routed experts, or above kKsplitRows rows: there an
// item is two tiles (16 gate rows, then their 16 up rows) on one activation
// operand, which halves the activation bytes a CU reads per weight byte.
// Each output element's arithmetic is the same either way.  Measured
// (paired A/B): MXFP4 16 rows -11.7 us; FP8 64 rows -19 to -25 us (ring
// depth 6), while FP8 from 5 to 16 rows lost 0.5 to 2.6 us and the 8-way
// expert-parallel share at 64 rows 15 us (a CU's jobs are then few, and its
// last chunks end further apart), so stream_geometry keeps FP8 layers with
// fewer than 32 (group, tile) pairs per CU at one tile.
__host__ __device__ inline int stream_ti(int T, int fmt) {
  return (stream_al(T) == 2 && fmt != 0) || T > kKsplitRows ? 16 : 8;
}
constexpr int kSpreadRows = 8;          // from this many rows (up to 8) each row is routed by one CU

// Workspace layout (byte offsets from the workspace base).
struct WsLayout {
  size_t flags, err, scores, picks, mid, total;
  int mid_ld;  // bf16 elements per (row, slot) line of mid
};

struct Params {
  // shape
  int H, I, Is, E, K, ng, kg, n_shared, T;
  int ef, ec;       // routed experts held here: [ef, ef + ec) (ec = E: all); weights indexed e - ef
  int routed_fmt, bias_bf16;
  double routed_scale;
  int hs;          // output rows per CU in down
  int ncu;         // workgroups launched (= CUs)
  int mid_ld;
  int lds_bytes;   // dynamic LDS size
  int rslots;      // routing scratch slots (one per wave that routes at once)
  int rsover;      // 1: the routing scratch may share LDS with the stream partials (no stream runs while routing)
  // stream geometry (see lds_offsets)
  int nrt_p;       // 16-row down tiles of a CU's slice, rounded up to 1, 2 or 4
  int kph;         // K-phases of a down sum: waves per down tile (8 / nrt_p); every
                   // down product is the sum of its K-phase partials in phase order
  int wpt;         // copies of the down products in LDS: kph up to kKsplitRows rows
                   // (one per K-phase), else 1 (each wave claims whole down jobs
                   // and adds their K-phase partials itself)
  int pitch;       // floats per (row, slot) line of the down products (16 * tiles)
  int cpj;         // columns per job (4 * AL); groups with more are split
  int pcols;       // columns of an up/gate partial tile (min(T, cpj))
  int ti, lti;     // intermediates per up/gate tile (stream_ti) and its log2
  int qcap;        // up/gate job entries of a CU (its share of the most jobs a batch can have)
  int dcap;        // down job entries (one per group and column tile, most a batch can have)
  // inputs
  const uint16_t* x;
  const uint16_t* router_w;
  const void* bias;
  const uint8_t* wgu;
  const void* sgu;
  const uint8_t* wd;
  const void* sd;
  const uint8_t* sh_wgu;
  const float* sh_sgu;
  const uint8_t* sh_wd;
  const float* sh_sd;
  // outputs
  uint16_t* out;
  int32_t* ids_out;
  float* w_out;
  union {
    int32_t* groups_out;       // groups mode
    const uint16_t* residual;  // forward: optional [T, H] bf16 added in the combine (NULL: none)
  };
  // workspace
  uint32_t* flags;
  uint32_t* err;
  double* scores;  // [T][E] score slots: two 64-bit words (tag, high half of s), (tag, low half)
  uint64_t* picks; // [T][K] routed picks above 8 rows: two 64-bit words (tag, expert), (tag, weight bits)
  uint16_t* mid;   // [T][K+1][mid_ld] bf16
  uint64_t* timeline;  // optional phase stamps ([ncu][64]); NULL unless built with MOE_TIMELINE
  // forward after an upstream producer: x is read only once *x_ready has
  // reached x_ready_value (wrap-around compare); NULL: x is ready at launch
  const uint32_t* x_ready;
  uint32_t x_ready_value;
  uint32_t x_spins;  // the wait's bound in polls
};

WsLayout ws_layout(int max_rows, int E, int K, int H, int I, int Is);
// Fills the stream geometry of p (T, K, E, I, Is, hs, ncu, n_shared set)
// and returns the LDS bytes it needs.
// fp8_tiles: the tiles of an FP8-routed instance whatever p.routed_fmt is
// (the unfused layout's shared-expert launches are FP8 instances).
size_t stream_geometry(Params& p, bool fp8_tiles = false);
// Launches the fused kernel instance for p and mode on device `dev` (the
// current device).  Returns hipErrorCooperativeLaunchTooLarge when one
// workgroup per CU with p's LDS size cannot be resident on this device.
hipError_t launch(const Params& p, int mode, hipStream_t stream, int dev);
// moe_forward / moe_forward_residual after their own argument checks:
// validates, carves the workspace ws (ws_bytes) and launches.
int forward_checked(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                    const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, void* stream,
                    const uint32_t* x_ready = nullptr, uint32_t x_ready_value = 0, uint32_t x_spins = 0);

// out[i] = bf16_RNE(a[i] + b[i]) for i < n (bf16 in, fp32 sum), on stream.
hipError_t launch_add(const uint16_t* a, const uint16_t* b, uint16_t* out, size_t n, hipStream_t stream);

// Records the HIP error behind a MOE_ERR_HIP return (moe_last_hip_error).
void set_last_hip(int e);
constexpr int kMaxDevices = 64;

}  // namespace moe
