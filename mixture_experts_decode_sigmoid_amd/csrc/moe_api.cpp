// moe_api.cpp -- host side of the C ABI in include/moe.h: argument
// validation, workspace carving and the launch.  No allocation, no host
// synchronisation (except moe_read_error, which is documented to wait).
#include "moe.h"
#include "moe_internal.h"

#include <string.h>

#include <atomic>
#include <mutex>

using namespace moe;

namespace {

thread_local int g_last_hip = 0;

constexpr int kNoRows = -1;  // fill(): valid call with rows == 0

struct DevInfo {
  int ncu = 0;
  size_t max_lds = 0;
};

// Device properties, cached per device id (read once under a lock; later
// reads see the published entry through the acquire load of `have`).
DevInfo dev_info(int dev) {
  static DevInfo cache[kMaxDevices];
  static std::atomic<bool> have[kMaxDevices];
  static std::mutex fill_lock;
  if (dev < 0 || dev >= kMaxDevices) return DevInfo{};
  if (!have[dev].load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> g(fill_lock);
    if (!have[dev].load(std::memory_order_relaxed)) {
      hipDeviceProp_t pr;
      if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return DevInfo{};
      cache[dev].ncu = pr.multiProcessorCount;
      cache[dev].max_lds = pr.sharedMemPerBlock;
      have[dev].store(true, std::memory_order_release);
    }
  }
  return cache[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_NULL;
  if (c->routed_fmt != MOE_FMT_FP8_B128 && c->routed_fmt != MOE_FMT_MXFP4) return MOE_ERR_FORMAT;
  if (c->shared_fmt != MOE_FMT_FP8_B128) return MOE_ERR_FORMAT;
  if (c->bias_dtype != MOE_BIAS_F32 && c->bias_dtype != MOE_BIAS_BF16) return MOE_ERR_FORMAT;
  if (c->hidden < 128 || c->hidden > 8192 || c->hidden % 128) return MOE_ERR_SHAPE;
  if (c->inter < 128 || c->inter > 4096 || c->inter % 128) return MOE_ERR_SHAPE;
  // MXFP4 experts stream 256 values of a row per item, and an up/gate job
  // needs at least one item for each of its 8 K-phases
  if (c->routed_fmt == MOE_FMT_MXFP4 && (c->hidden % 256 || c->hidden < 2048 || c->inter % 256))
    return MOE_ERR_SHAPE;
  if (c->n_shared != 0 && c->n_shared != 1) return MOE_ERR_SHAPE;
  if (c->n_shared && (c->shared_inter < 128 || c->shared_inter > 4096 || c->shared_inter % 128))
    return MOE_ERR_SHAPE;
  if (c->n_experts < 1 || c->n_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->n_experts) return MOE_ERR_SHAPE;
  if (c->n_group < 1 || c->n_group > kMaxGroups || c->n_experts % c->n_group) return MOE_ERR_SHAPE;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_SHAPE;
  if (c->n_group > 1) {
    const int gsz = c->n_experts / c->n_group;
    if (gsz < 2 || c->topk_group * gsz < c->top_k) return MOE_ERR_SHAPE;
  }
  if (!(c->routed_scale == c->routed_scale)) return MOE_ERR_SHAPE;
  if (c->max_rows < 1 || c->max_rows > kMaxRows) return MOE_ERR_ROWS;
  if (c->expert_count < 0 || c->expert_first < 0) return MOE_ERR_SHAPE;
  if (c->expert_count == 0 ? c->expert_first != 0 : c->expert_first > c->n_experts - c->expert_count)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

int check_weights(const moe_config* c, const moe_weights* w, bool need_experts) {
  if (!w) return MOE_ERR_NULL;
  if (!w->router_w || !w->bias) return MOE_ERR_NULL;
  if (need_experts) {
    if (!w->w_gate_up || !w->s_gate_up || !w->w_down || !w->s_down) return MOE_ERR_NULL;
    if (c->n_shared && (!w->sh_w_gate_up || !w->sh_s_gate_up || !w->sh_w_down || !w->sh_s_down))
      return MOE_ERR_NULL;
  }
  const void* ps[] = {w->router_w, w->bias, w->w_gate_up, w->s_gate_up, w->w_down, w->s_down,
                      w->sh_w_gate_up, w->sh_s_gate_up, w->sh_w_down, w->sh_s_down};
  const int n = need_experts ? 10 : 2;
  for (int i = 0; i < n; ++i)
    if (ps[i] && !aligned16(ps[i])) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int hs_for(int H, int ncu) { return (H + ncu - 1) / ncu; }

int fill(const moe_config* c, const moe_weights* w, const uint16_t* x, int rows, void* ws,
         size_t ws_bytes, Params& p, int mode, int& dev) {
  int rc = check_cfg(c);
  if (rc) return rc;
  rc = check_weights(c, w, mode == kModeForward);
  if (rc) return rc;
  if (rows < 0 || rows > c->max_rows) return MOE_ERR_ROWS;
  if (rows == 0) return kNoRows;  // a no-op: x, out and ws may be NULL
  if (!x || !ws) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(ws)) return MOE_ERR_ALIGN;
  const WsLayout L = ws_layout(c->max_rows, c->n_experts, c->top_k, c->hidden, c->inter,
                               c->n_shared ? c->shared_inter : 0);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const DevInfo d = dev_info(dev);
  if (d.ncu <= 0) {
    g_last_hip = (int)hipErrorNoDevice;
    return MOE_ERR_HIP;
  }
  if (d.ncu > 1024) return MOE_ERR_SHAPE;
  const int hs = hs_for(c->hidden, d.ncu);
  if (hs > kMaxSlice) return MOE_ERR_SHAPE;
  memset(&p, 0, sizeof p);
  p.H = c->hidden;
  p.I = c->inter;
  p.Is = c->n_shared ? c->shared_inter : 0;
  p.E = c->n_experts;
  p.ef = c->expert_first;
  p.ec = c->expert_count ? c->expert_count : c->n_experts;
  p.K = c->top_k;
  p.ng = c->n_group;
  p.kg = c->topk_group;
  p.n_shared = c->n_shared;
  p.T = rows;
  p.routed_fmt = c->routed_fmt;
  p.bias_bf16 = c->bias_dtype == MOE_BIAS_BF16;
  p.routed_scale = (double)c->routed_scale;
  p.hs = hs;
  p.ncu = d.ncu;
  p.mid_ld = L.mid_ld;
  // up to 8 rows every wave may route a row; above, a forward call routes
  // row r on wave r / ncu of CU r mod ncu (or on wave 7, while the other
  // waves stream), and the routing-only calls route on every wave of one CU
  // with no stream running
  if (rows <= kWaves || mode != kModeForward) {
    p.rslots = kWaves;
    p.rsover = rows > kWaves;
  } else {
    p.rslots = (rows + d.ncu - 1) / d.ncu;
    p.rsover = 0;
  }
  size_t lds = stream_geometry(p);
  if (lds > d.max_lds) return MOE_ERR_SHAPE;
  if (lds < (size_t)kMinLds) lds = kMinLds;
  p.lds_bytes = (int)lds;
  p.x = x;
  p.router_w = w->router_w;
  p.bias = w->bias;
  p.wgu = w->w_gate_up;
  p.sgu = w->s_gate_up;
  p.wd = w->w_down;
  p.sd = w->s_down;
  p.sh_wgu = w->sh_w_gate_up;
  p.sh_sgu = w->sh_s_gate_up;
  p.sh_wd = w->sh_w_down;
  p.sh_sd = w->sh_s_down;
  char* base = (char*)ws;
  p.flags = (uint32_t*)(base + L.flags);
  p.err = (uint32_t*)(base + L.err);
  p.scores = (double*)(base + L.scores);
  p.picks = (uint64_t*)(base + L.picks);
  p.mid = (uint16_t*)(base + L.mid);
#ifdef MOE_TIMELINE
  p.timeline = (uint64_t*)(base + L.total);  // callers of a timeline build add 1024*16*8 bytes
  if (ws_bytes < L.total + 1024 * 16 * 8) return MOE_ERR_WORKSPACE;
#endif
  return MOE_OK;
}

int do_launch(const Params& p, int mode, void* stream, int dev) {
  hipError_t e = launch(p, mode, (hipStream_t)stream, dev);
  if (e == hipErrorCooperativeLaunchTooLarge) return MOE_ERR_LAUNCH;
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace

void moe::set_last_hip(int e) { g_last_hip = e; }

int moe::forward_checked(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                         const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, void* stream,
                         const uint32_t* x_ready, uint32_t x_ready_value, uint32_t x_spins) {
  Params p;
  int dev = 0;
  int rc = fill(cfg, w, x, rows, ws, ws_bytes, p, kModeForward, dev);
  if (rc == kNoRows) return MOE_OK;
  if (rc) return rc;
  if (!out) return MOE_ERR_NULL;
  if (!aligned16(out)) return MOE_ERR_ALIGN;
  const size_t nb = (size_t)rows * cfg->hidden * 2;
  const char *xo = (const char*)x, *oo = (const char*)out;
  if (rows > 0 && xo < oo + nb && oo < xo + nb) return MOE_ERR_ALIAS;
  if (residual) {
    // the residual may be out itself (each element is read, then written,
    // by one thread) but may not overlap it otherwise
    const char* ro = (const char*)residual;
    if (ro != oo && ro < oo + nb && oo < ro + nb) return MOE_ERR_ALIAS;
  }
  if (rows == 0) return MOE_OK;
  p.out = out;
  p.residual = residual;
  p.x_ready = x_ready;
  p.x_ready_value = x_ready_value;
  p.x_spins = x_spins ? x_spins : 400000u;
  return do_launch(p, kModeForward, stream, dev);
}

extern "C" {

int moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  int rc = check_cfg(cfg);
  if (rc) return rc;
  *bytes = ws_layout(cfg->max_rows, cfg->n_experts, cfg->top_k, cfg->hidden, cfg->inter,
                     cfg->n_shared ? cfg->shared_inter : 0).total;
  return MOE_OK;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_ERR_NULL;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  const WsLayout L = ws_layout(1, 1, 1, 128, 128, 0);
  if (ws_bytes < L.scores) return MOE_ERR_WORKSPACE;
  // the whole workspace: flags, error word and the tagged score slots
  hipError_t e = hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  Params p;
  int dev = 0;
  int rc = fill(cfg, w, x, rows, ws, ws_bytes, p, kModeRoute, dev);
  if (rc == kNoRows) return MOE_OK;
  if (rc) return rc;
  if (!topk_ids || !topk_w) return MOE_ERR_NULL;
  if (rows == 0) return MOE_OK;
  p.ids_out = topk_ids;
  p.w_out = topk_w;
  return do_launch(p, kModeRoute, stream, dev);
}

int moe_groups(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
               int32_t* groups_out, void* ws, size_t ws_bytes, void* stream) {
  Params p;
  int dev = 0;
  int rc = fill(cfg, w, x, rows, ws, ws_bytes, p, kModeGroups, dev);
  if (rc == kNoRows) return MOE_OK;
  if (rc) return rc;
  if (!groups_out) return MOE_ERR_NULL;
  if (rows == 0) return MOE_OK;
  p.groups_out = groups_out;
  return do_launch(p, kModeGroups, stream, dev);
}

int moe_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  return forward_checked(cfg, w, x, rows, nullptr, out, ws, ws_bytes, stream);
}

int moe_forward_residual(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                         const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (rows > 0 && !residual) return MOE_ERR_NULL;
  return forward_checked(cfg, w, x, rows, residual, out, ws, ws_bytes, stream);
}

int moe_forward_prefill(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows, uint16_t* out,
                        void* ws, size_t ws_bytes, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (rows < 0) return MOE_ERR_ROWS;
  if (rows == 0) return MOE_OK;
  if (!x || !out) return MOE_ERR_NULL;
  const size_t nb = (size_t)rows * cfg->hidden * 2;
  const char *xo = (const char*)x, *oo = (const char*)out;
  if (xo < oo + nb && oo < xo + nb) return MOE_ERR_ALIAS;
  for (int r0 = 0; r0 < rows; r0 += cfg->max_rows) {
    const int n = rows - r0 < cfg->max_rows ? rows - r0 : cfg->max_rows;
    const size_t off = (size_t)r0 * cfg->hidden;
    rc = forward_checked(cfg, w, x + off, n, nullptr, out + off, ws, ws_bytes, stream);
    if (rc) return rc;
  }
  return MOE_OK;
}

int moe_forward_unfused(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows, uint16_t* out,
                        uint16_t* tmp_routed, uint16_t* tmp_shared, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!cfg->n_shared) return MOE_ERR_SHAPE;
  if (rows == 0) return rows <= cfg->max_rows ? MOE_OK : MOE_ERR_ROWS;
  if (!out || !tmp_routed || !tmp_shared) return MOE_ERR_NULL;
  if (!aligned16(out) || !aligned16(tmp_routed) || !aligned16(tmp_shared)) return MOE_ERR_ALIGN;
  if (rows > 0) {
    const size_t nb = (size_t)rows * cfg->hidden * 2;
    const char* b[4] = {(const char*)x, (const char*)out, (const char*)tmp_routed, (const char*)tmp_shared};
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (b[i] < b[j] + nb && b[j] < b[i] + nb) return MOE_ERR_ALIAS;
  }
  // 1: the routed experts alone (the fused pass of a layer without a shared expert)
  moe_config routed = *cfg;
  routed.n_shared = 0;
  rc = forward_checked(&routed, w, x, rows, nullptr, tmp_routed, ws, ws_bytes, stream);
  if (rc) return rc;
  // 2, 3: the shared expert's gate/up, then its down
  Params p;
  int dev = 0;
  rc = fill(cfg, w, x, rows, ws, ws_bytes, p, kModeForward, dev);
  if (rc == kNoRows) return MOE_OK;
  if (rc) return rc;
  p.out = tmp_shared;
  // the shared-expert launches are FP8 instances: their tile size is the
  // FP8 kernels' whatever the routed format
  {
    size_t lds = stream_geometry(p, true);
    if (lds < (size_t)kMinLds) lds = kMinLds;
    p.lds_bytes = (int)lds;
  }
  rc = do_launch(p, kModeSharedUp, stream, dev);
  if (rc) return rc;
  rc = do_launch(p, kModeSharedDown, stream, dev);
  if (rc) return rc;
  // 4: the add
  const hipError_t e = launch_add(tmp_routed, tmp_shared, out, (size_t)rows * cfg->hidden, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_forward_after(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int rows,
                      const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes,
                      const uint32_t* x_ready, uint32_t x_ready_value, uint32_t max_polls, void* stream) {
  if (rows > 0 && !x_ready) return MOE_ERR_NULL;
  if (x_ready && ((uintptr_t)x_ready & 3u)) return MOE_ERR_ALIGN;
  return forward_checked(cfg, w, x, rows, residual, out, ws, ws_bytes, stream, x_ready, x_ready_value, max_polls);
}

int moe_read_error(void* ws, void* stream, uint32_t* bits) {
  if (!ws || !bits) return MOE_ERR_NULL;
  const WsLayout L = ws_layout(1, 1, 1, 128, 128, 0);
  uint32_t* err = (uint32_t*)((char*)ws + L.err);
  hipError_t e = hipMemcpyAsync(bits, err, 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemsetAsync(err, 0, 4, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "sizes outside what the kernels support";
    case MOE_ERR_FORMAT: return "unknown weight format or bias dtype";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_ROWS: return "rows out of range (0..max_rows, max_rows <= 64)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ALIAS: return "out overlaps x, or the residual overlaps out without being it";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_LAUNCH: return "one workgroup per CU at this LDS size cannot be resident on this device";
    default: return "unknown error code";
  }
}

int moe_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
