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

enum Mode { kModeForward = 0, kModeRoute = 1, kModeGroups = 2, kModeForwardRes = 3 };  // 3: kernel only (wide stream with a residual)

// Workspace layout (byte offsets from the workspace base).
struct WsLayout {
  size_t flags, err, scores, mid, total;
  int mid_ld;  // bf16 elements per (row, slot) line of mid
};

struct Params {
  // shape
  int H, I, Is, E, K, ng, kg, n_shared, T;
  int routed_fmt, bias_bf16;
  double routed_scale;
  int hs;          // output rows per CU in down
  int ncu;         // workgroups launched (= CUs)
  int mid_ld;
  int lds_bytes;   // dynamic LDS size
  // stream geometry (see lds_offsets): narrow = per-wave partials in LDS
  int narrow;      // 1: batches of at most 16 rows whose partials fit in LDS
  int nrt_p;       // 16-row down tiles of a CU's slice, rounded up to 1, 2 or 4
  int wpt;         // waves per down tile (8 / nrt_p); they split its K-blocks
  int pitch;       // floats per (row, slot) line of the down products (16 * tiles)
  int qcap;        // narrow: up/gate job entries of a CU (its share of the most jobs a batch can have)
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
  uint16_t* mid;   // [T][K+1][mid_ld] bf16
  uint64_t* timeline;  // optional phase stamps ([ncu][64]); NULL unless built with MOE_TIMELINE
};

WsLayout ws_layout(int max_rows, int E, int K, int H, int I, int Is);
// Fills the stream geometry of p (T, K, E, I, Is, hs, ncu set) for the
// narrow (narrow = 1) or wide layout and returns the LDS bytes it needs.
size_t stream_geometry(Params& p, int narrow);
// Launches the fused kernel instance for p and mode on device `dev` (the
// current device).  Returns hipErrorCooperativeLaunchTooLarge when one
// workgroup per CU with p's LDS size cannot be resident on this device.
hipError_t launch(const Params& p, int mode, hipStream_t stream, int dev);
// The forward of the wide stream with a residual (moe_kernels_res.hip).
hipError_t launch_res_wide(const Params& p, hipStream_t stream, int dev);
// moe_forward / moe_forward_residual after their own argument checks:
// validates, carves the workspace ws (ws_bytes) and launches.
int forward_checked(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                    const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

// Records the HIP error behind a MOE_ERR_HIP return (moe_last_hip_error).
void set_last_hip(int e);
constexpr int kMaxDevices = 64;

}  // namespace moe
