// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (no GPU needed): configuration and argument
// validation, workspace sizing, no-op calls and every error string.  Built
// with the host compiler against the library's device objects; prints "ok".
#include <stdio.h>
#include <string.h>

#include "moe.h"

static moe_config v3(void) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.hidden = 7168; c.inter = 2048; c.shared_inter = 2048; c.n_experts = 256; c.top_k = 8;
  c.n_group = 8; c.topk_group = 4; c.n_shared = 1; c.routed_scale = 2.5f;
  c.routed_fmt = MOE_FMT_FP8_B128; c.shared_fmt = MOE_FMT_FP8_B128; c.bias_dtype = MOE_BIAS_F32;
  c.max_rows = 64;
  return c;
}

#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main(void) {
  size_t n = 0;
  moe_config c = v3();
  EXPECT(moe_workspace_size(&c, &n) == MOE_OK && n > 0);
  // every field out of range once
  struct { int* f; int bad; } cases[] = {
      {&c.hidden, 100}, {&c.inter, 0}, {&c.shared_inter, 64}, {&c.n_experts, 300}, {&c.top_k, 9},
      {&c.n_group, 7}, {&c.topk_group, 9}, {&c.n_shared, 2}, {&c.routed_fmt, 5}, {&c.shared_fmt, 1},
      {&c.bias_dtype, 3}, {&c.max_rows, 65}, {&c.expert_first, 300}, {&c.expert_count, -1}};
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    moe_config b = v3();
    *(int*)((char*)&b + ((char*)cases[i].f - (char*)&c)) = cases[i].bad;
    EXPECT(moe_workspace_size(&b, &n) != MOE_OK);
  }
  EXPECT(moe_workspace_size(NULL, &n) == MOE_ERR_NULL);
  // sizes over the whole accepted range of rows and shapes
  for (int rows = 1; rows <= 64; rows += 7) {
    moe_config b = v3();
    b.max_rows = rows;
    EXPECT(moe_workspace_size(&b, &n) == MOE_OK);
  }
  moe_config m = v3();
  m.routed_fmt = MOE_FMT_MXFP4;
  m.bias_dtype = MOE_BIAS_BF16;
  EXPECT(moe_workspace_size(&m, &n) == MOE_OK);
  m.hidden = 2176;
  EXPECT(moe_workspace_size(&m, &n) == MOE_ERR_SHAPE);
  // calls that fail validation or do nothing never touch the device
  moe_weights w;
  memset(&w, 0, sizeof w);
  EXPECT(moe_forward(&c, &w, NULL, 0, NULL, NULL, 0, NULL) == MOE_ERR_NULL);
  w.router_w = (const uint16_t*)0x10000; w.bias = (const void*)0x10000;
  w.w_gate_up = (const uint8_t*)0x10000; w.s_gate_up = (const void*)0x10000;
  w.w_down = (const uint8_t*)0x10000; w.s_down = (const void*)0x10000;
  w.sh_w_gate_up = (const uint8_t*)0x10000; w.sh_s_gate_up = (const float*)0x10000;
  w.sh_w_down = (const uint8_t*)0x10000; w.sh_s_down = (const float*)0x10000;
  EXPECT(moe_forward(&c, &w, NULL, 0, NULL, NULL, 0, NULL) == MOE_OK);
  EXPECT(moe_forward(&c, &w, (const uint16_t*)0x1000, -1, NULL, NULL, 0, NULL) == MOE_ERR_ROWS);
  EXPECT(moe_forward(&c, &w, (const uint16_t*)0x1000, 65, NULL, NULL, 0, NULL) == MOE_ERR_ROWS);
  EXPECT(moe_forward(&c, &w, (const uint16_t*)0x1008, 1, (uint16_t*)0x2000, (void*)0x4000, 1u << 30, NULL) ==
         MOE_ERR_ALIGN);
  EXPECT(moe_forward(&c, &w, (const uint16_t*)0x1000, 1, (uint16_t*)0x4000, (void*)0x8000, 16, NULL) ==
         MOE_ERR_WORKSPACE);
  EXPECT(moe_forward_prefill(&c, &w, (const uint16_t*)0x1000, 0, NULL, NULL, 0, NULL) == MOE_OK);
  EXPECT(moe_forward_prefill(&c, &w, (const uint16_t*)0x1000, 100, (uint16_t*)0x1040, (void*)0x4000, 1u << 30,
                             NULL) == MOE_ERR_ALIAS);
  EXPECT(moe_probe_stream_read(NULL, 1, NULL, 1, NULL) == MOE_ERR_NULL);
  EXPECT(moe_pack_mxfp4_scales(NULL, (uint8_t*)0x1000, 16, 256, NULL) == MOE_ERR_NULL);
  EXPECT(moe_pack_mxfp4_scales((const uint8_t*)0x1008, (uint8_t*)0x2000, 16, 256, NULL) == MOE_ERR_ALIGN);
  EXPECT(moe_pack_mxfp4_scales((const uint8_t*)0x1000, (uint8_t*)0x2000, 15, 256, NULL) == MOE_ERR_SHAPE);
  EXPECT(moe_pack_mxfp4_scales((const uint8_t*)0x1000, (uint8_t*)0x2000, 16, 128, NULL) == MOE_ERR_SHAPE);
  EXPECT(moe_pack_mxfp4_scales((const uint8_t*)0x1000, (uint8_t*)0x1040, 16, 256, NULL) == MOE_ERR_ALIAS);
  for (int code = -2; code <= 12; ++code) EXPECT(moe_strerror(code) != NULL && moe_strerror(code)[0]);
  printf("ok\n");
  return 0;
}
