// Drives the host side of the C-ABI library -- argument and shape checks,
// workspace sizing, status strings, the no-device path -- for a build whose
// host code runs under AddressSanitizer and UndefinedBehaviorSanitizer (the
// device code is built as usual and never launched: device pointers here are
// fake, aligned addresses the host never dereferences).  Any out-of-bounds
// access or undefined operation in the host code aborts the run.  Prints
// "host api checks ok" and exits 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <climits>
#include <initializer_list>

#include "coli_moe.h"

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);      \
      exit(1);                                                               \
    }                                                                        \
  } while (0)

template <class T = void>
static T *fake(uintptr_t a) { return reinterpret_cast<T *>(a); }

static coli_router_cfg router(int E, int k, int G, int TG, float p = 0.0f) {
  coli_router_cfg c;
  c.n_experts = E; c.top_k = k; c.n_group = G; c.topk_group = TG;
  c.norm_topk_prob = 1; c.routed_scaling_factor = 2.5f; c.expert_top_p = p; c.top_p_renorm = 1;
  return c;
}

static coli_moe_layer layer(int H = 6144, int I = 2048, int q = 4, int E = 256, int k = 8,
                            int G = 8, int TG = 4) {
  coli_moe_layer L;
  memset(&L, 0, sizeof L);
  L.hidden = H; L.inter = I; L.qtype = q;
  L.router = router(E, k, G, TG);
  const uint8_t **u8[] = {&L.w_gate, &L.w_up, &L.w_down, &L.sh_gate, &L.sh_up, &L.sh_down};
  const float **f32[] = {&L.gate_w, &L.gate_bias, &L.s_gate, &L.s_up, &L.s_down,
                         &L.sh_s_gate, &L.sh_s_up, &L.sh_s_down};
  uintptr_t a = 0x10000;
  for (auto p : u8) { *p = fake<const uint8_t>(a); a += 0x10000; }
  for (auto p : f32) { *p = fake<const float>(a); a += 0x10000; }
  return L;
}

int main() {
  CHECK(coli_abi_version() == COLI_ABI_VERSION);
  const int codes[] = {0, 1, 2, 3, 4, 5, -1, 99, INT_MIN, INT_MAX};
  for (int s : codes) CHECK(coli_status_str(s) != nullptr);
  CHECK(strcmp(coli_status_str(-1), "unknown status") == 0);

  // elementwise entry points: malformed arguments
  CHECK(coli_quant_pack(3, fake<float>(16), 4, 32, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_quant_pack(4, fake<float>(16), 4, 48, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_quant_pack(4, fake<float>(16), INT64_MAX, INT64_MAX & ~31ll, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_UNSUPPORTED);
  CHECK(coli_quant_pack_fp8(4, fake<uint8_t>(16), fake<float>(16), -1, 32, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_quant_pack_fp8(4, fake<uint8_t>(16), fake<float>(16), INT64_MAX, INT64_MAX & ~31ll, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_UNSUPPORTED);
  CHECK(coli_gemv_f32act(4, fake<uint8_t>(16), fake<float>(16), 4, 16384 + 32, fake<float>(16), fake<float>(16), nullptr) == COLI_ERR_UNSUPPORTED);
  CHECK(coli_gemv_f32act(2, fake<uint8_t>(16), fake<float>(16), 4, 32, fake<float>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_gemv_f32act(4, fake<uint8_t>(16), fake<float>(16), INT64_MAX, 64, fake<float>(16), fake<float>(16), nullptr) == COLI_ERR_UNSUPPORTED);
  CHECK(coli_quant_act_q8_0(fake<float>(16), 1, 33, fake<int8_t>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_quant_act_q8_0(fake<float>(16), INT_MAX, INT_MAX & ~31, fake<int8_t>(16), fake<float>(16), nullptr) == COLI_ERR_UNSUPPORTED);
  CHECK(coli_moe_logits(fake<float>(16), fake<float>(16), 1, 0, 64, fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_logits(fake<float>(16), fake<float>(16), INT_MAX, INT_MAX, INT_MAX, fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);

  // routing and dispatch configurations
  const coli_router_cfg bad_cfgs[] = {router(256, 8, 7, 4), router(256, 40, 8, 8), router(16, 5, 4, 1),
                                      router(0, 1, 1, 1), router(2048, 8, 8, 4), router(256, 8, 8, 9),
                                      router(256, 0, 8, 4), router(INT_MAX, INT_MAX, 1, 1)};
  for (const coli_router_cfg &c : bad_cfgs)
    CHECK(coli_moe_route(&c, fake<float>(16), nullptr, 1, fake<int32_t>(16), fake<float>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_dispatch(fake<int32_t>(16), 4, 0, 16, fake<int32_t>(16), fake<int32_t>(16), fake<int32_t>(16),
                          fake<int32_t>(16), fake<int32_t>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_dispatch(fake<int32_t>(16), INT_MAX, 32, 256, fake<int32_t>(16), fake<int32_t>(16), fake<int32_t>(16),
                          fake<int32_t>(16), fake<int32_t>(16), nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_debug_qgemv_blocks(4, fake<uint8_t>(16), 4, 96, fake<int8_t>(16), 1, fake<int32_t>(16), nullptr) == COLI_ERR_INVALID_ARG);

  // workspace sizing over the whole token range and every container
  for (int q : {8, 4, 2}) {
    for (int E : {16, 256, 1024}) {
      coli_moe_layer L = layer(8192, 8192, q, E, 8, 8, 4);
      size_t prev = 0;
      for (int32_t T : {1, 2, 3, 64, 512, 4096, 65536, 1 << 20, INT_MAX / 64, INT_MAX}) {
        const size_t b = coli_moe_workspace_bytes(&L, T);
        CHECK(b == 0 || (b % 256 == 0 && b > prev));
        if (b) prev = b;
      }
      CHECK(coli_moe_workspace_bytes(&L, 0) == 0 || coli_moe_workspace_bytes(&L, 0) % 256 == 0);
      CHECK(coli_moe_workspace_bytes(&L, -1) == 0);
    }
  }
  CHECK(coli_moe_workspace_bytes(nullptr, 1) == 0);

  // forward: every layer-shape check, workspace checks
  coli_moe_layer good = layer();
  const size_t ws = coli_moe_workspace_bytes(&good, 1);
  CHECK(ws > COLI_WORKSPACE_COUNTER_BYTES);
  float *x = fake<float>(0x100000), *y = fake<float>(0x200000);
  void *wsp = fake(0x300000);
  CHECK(coli_moe_forward(&good, x, 1, nullptr, y, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == COLI_ERR_WORKSPACE);
  CHECK(coli_moe_forward(&good, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws - 1, nullptr) == COLI_ERR_WORKSPACE);
  CHECK(coli_moe_forward(&good, x, 1, nullptr, y, nullptr, nullptr, nullptr, fake(0x300010), ws, nullptr) == COLI_ERR_WORKSPACE);
  CHECK(coli_moe_forward(&good, x, -1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_forward(nullptr, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  const coli_moe_layer bad_layers[] = {layer(6000), layer(6144, 100), layer(6144, 2048, 3),
                                       layer(6144, 2048, 4, 1025, 8, 1, 1), layer(16384),
                                       layer(INT_MAX & ~63, INT_MAX & ~63), layer(-64, 2048),
                                       layer(6144, 2048, 4, 256, 40, 8, 8)};
  for (const coli_moe_layer &L : bad_layers) {
    CHECK(coli_moe_workspace_bytes(&L, 1) == 0);
    CHECK(coli_moe_forward(&L, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
    CHECK(coli_moe_forward_noalloc(&L, x, 1, nullptr, y, nullptr, nullptr, nullptr, nullptr, nullptr) == COLI_ERR_INVALID_ARG);
  }
  coli_moe_layer s = layer();
  s.w_down = nullptr;
  CHECK(coli_moe_forward(&s, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  s = layer();
  s.w_up = fake<const uint8_t>(0x10008);
  CHECK(coli_moe_forward(&s, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  s = layer();
  s.gate_w = nullptr;
  CHECK(coli_moe_forward(&s, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  // the no-allocation variant rejects a batch beyond its static scratch
  CHECK(coli_moe_forward_noalloc(&good, x, INT_MAX, nullptr, y, nullptr, nullptr, nullptr, nullptr, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_forward_noalloc(&good, x, 1 << 20, nullptr, y, nullptr, nullptr, nullptr, nullptr, nullptr) == COLI_ERR_UNSUPPORTED);
  // workspace status: null, misaligned, bad output pointer
  CHECK(coli_moe_workspace_status(nullptr, fake<int32_t>(16), 0, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_workspace_status(fake(0x300010), fake<int32_t>(16), 0, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_workspace_status(wsp, nullptr, 1, nullptr) == COLI_ERR_INVALID_ARG);
  // debug entry points
  CHECK(coli_debug_stream_read(fake(0x300000), 15, fake<uint32_t>(16), nullptr, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_debug_stream_read(nullptr, 16, fake<uint32_t>(16), nullptr, nullptr) == COLI_ERR_INVALID_ARG);

  // expert cache: layouts over the whole size range, malformed descriptors,
  // host tiers outside any coli_host_alloc allocation
  for (int E : {1, 16, 256, 1024, 1025, 0, -5}) {
    for (int S : {0, 1, 8, E, E + 1}) {
      coli_expert_cache_layout lo;
      const coli_status r = coli_expert_cache_layout_of(E, S, &lo);
      if (E >= 1 && E <= 1024 && S >= 1 && S <= E) {
        CHECK(r == COLI_OK && lo.total % 256 == 0 && lo.copy_list + (size_t)S * 8 <= lo.total);
      } else {
        CHECK(r == COLI_ERR_INVALID_ARG);
      }
    }
  }
  coli_expert_cache C;
  memset(&C, 0, sizeof C);
  C.n_experts = 256;
  C.n_slots = 32;
  C.host_w_gate = fake<const uint8_t>(0x800000);
  C.host_w_up = fake<const uint8_t>(0x900000);
  C.host_w_down = fake<const uint8_t>(0xA00000);
  C.host_s_gate = fake<const float>(0xB00000);
  C.host_s_up = fake<const float>(0xC00000);
  C.host_s_down = fake<const float>(0xD00000);
  C.state = fake(0x400010);
  CHECK(coli_expert_cache_init(&C, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_expert_cache_init(nullptr, nullptr) == COLI_ERR_INVALID_ARG);
  C.state = fake(0x400000);
  CHECK(coli_moe_forward_cached(&good, &C, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_expert_cache_repin(&C, &good, 4, nullptr) == COLI_ERR_INVALID_ARG);
  C.n_pinned = 32;
  CHECK(coli_moe_forward_cached(&good, &C, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_moe_forward_cached(&good, nullptr, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_INVALID_ARG);
  CHECK(coli_host_free(nullptr) == COLI_OK);
  CHECK(coli_host_free(fake(0x12345000)) == COLI_ERR_INVALID_ARG);
  void *hp = nullptr;
  CHECK(coli_host_alloc(0, &hp) == COLI_ERR_INVALID_ARG);

  // with no device present, a well-formed call reports a device error
  const char *vis = getenv("COLI_EXPECT_NO_DEVICE");
  if (vis && vis[0] == '1') {
    CHECK(coli_moe_forward(&good, x, 1, nullptr, y, nullptr, nullptr, nullptr, wsp, ws, nullptr) == COLI_ERR_DEVICE);
    CHECK(coli_quant_pack(4, fake<float>(16), 4, 32, fake<uint8_t>(16), fake<float>(16), nullptr) == COLI_ERR_DEVICE);
    CHECK(coli_host_alloc(4096, &hp) == COLI_ERR_DEVICE && hp == nullptr);
  }
  printf("host api checks ok\n");
  return 0;
}
