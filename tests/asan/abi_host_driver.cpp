// Host-side exercise of the C ABI for an AddressSanitizer build: every call
// here returns before any HIP call (no GPU needed).  Exits non-zero on an
// unexpected status; the sanitizer aborts on a memory error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "flint_moe.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static flint_moe_config base_config() {
  flint_moe_config c;
  std::memset(&c, 0, sizeof c);
  c.hidden = 2048;
  c.n_experts = 256;
  c.top_k = 6;
  c.inter = 512;
  c.max_tokens = 8;
  c.renormalize = 1;
  c.routed_scale = 1.0f;
  c.format = FLINT_W_BF16;
  return c;
}

template <class T>
static T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }

static flint_moe_weights fake_weights() {
  flint_moe_weights w;
  std::memset(&w, 0, sizeof w);
  w.router_w = fake<const uint16_t>(1u << 20);
  w.routed.w13 = fake<const void>(1u << 22);
  w.routed.w2 = fake<const void>(1u << 23);
  w.shared.w13 = fake<const void>(1u << 24);
  w.shared.w2 = fake<const void>(1u << 25);
  return w;
}

int main() {
  // Status strings and NULL-safe calls.
  for (int s = 0; s <= 5; ++s) EXPECT(flint_moe_status_string((flint_status)s) != nullptr);
  EXPECT(std::strlen(flint_moe_last_error(nullptr)) == 0);
  flint_moe_destroy(nullptr);
  flint_mlp_destroy(nullptr);
  EXPECT(flint_moe_workspace_bytes(nullptr, 4) == 0);

  // init: rejected configurations.
  flint_moe_ctx* ctx = nullptr;
  EXPECT(flint_moe_init(nullptr, &ctx) == FLINT_ERR_INVALID_ARG);
  flint_moe_config c = base_config();
  EXPECT(flint_moe_init(&c, nullptr) == FLINT_ERR_INVALID_ARG);
  c.hidden = 4096;
  EXPECT(flint_moe_init(&c, &ctx) == FLINT_ERR_UNSUPPORTED);
  c = base_config();
  c.top_k = 9;   // more than the kernels are built for
  EXPECT(flint_moe_init(&c, &ctx) == FLINT_ERR_UNSUPPORTED);
  c = base_config();
  c.n_experts = 4;
  c.top_k = 5;   // more than there are experts
  EXPECT(flint_moe_init(&c, &ctx) == FLINT_ERR_INVALID_ARG);
  c = base_config();
  c.n_experts = 0;
  EXPECT(flint_moe_init(&c, &ctx) == FLINT_ERR_INVALID_ARG);
  c = base_config();
  c.max_tokens = 0;
  EXPECT(flint_moe_init(&c, &ctx) == FLINT_ERR_INVALID_ARG);
  c = base_config();
  c.format = 7;
  EXPECT(flint_moe_init(&c, &ctx) != FLINT_OK);
  EXPECT(ctx == nullptr);

  // A valid context for every batch size class, both formats.
  for (int fmt = 0; fmt < 2; ++fmt) {
    for (int max_t : {1, 8, 64, 65, 8192}) {
      c = base_config();
      c.format = fmt;
      c.max_tokens = max_t;
      ctx = nullptr;
      EXPECT(flint_moe_init(&c, &ctx) == FLINT_OK && ctx != nullptr);
      if (!ctx) continue;
      for (int T : {1, 2, 8, 9, 64, 65, 300, 8192}) {
        if (T > max_t) break;
        const size_t n = flint_moe_workspace_bytes(ctx, T);
        EXPECT(n >= FLINT_MOE_WS_HEADER_BYTES);
        flint_moe_ws_layout lay;
        EXPECT(flint_moe_workspace_layout(ctx, T, &lay) == FLINT_OK && lay.total_bytes == n);
      }
      EXPECT(flint_moe_workspace_bytes(ctx, 0) == 0);

      // forward: host-side rejections (fake device pointers are never touched).
      flint_moe_weights w = fake_weights();
      const int T = max_t < 4 ? max_t : 4;
      const size_t need = flint_moe_workspace_bytes(ctx, T);
      const uint16_t* x = fake<const uint16_t>(1ull << 30);
      uint16_t* out = fake<uint16_t>(1ull << 31);
      void* ws = fake<void>(1ull << 32);
      EXPECT(flint_moe_forward(ctx, &w, x, -1, out, nullptr, nullptr, ws, need, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      EXPECT(flint_moe_forward(ctx, &w, x, max_t + 1, out, nullptr, nullptr, ws, need, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      EXPECT(std::strlen(flint_moe_last_error(ctx)) > 0);
      EXPECT(flint_moe_forward(ctx, &w, nullptr, T, out, nullptr, nullptr, ws, need, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      EXPECT(flint_moe_forward(ctx, &w, x + 1, T, out, nullptr, nullptr, ws, need, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      if (fmt == FLINT_W_BF16)   // (NVFP4: the missing scales are reported first)
        EXPECT(flint_moe_forward(ctx, &w, x, T, out, nullptr, nullptr, ws, need - 1, nullptr) ==
               FLINT_ERR_WORKSPACE);
      EXPECT(flint_moe_forward(ctx, &w, x, T, fake<uint16_t>((1ull << 30) + 64), nullptr, nullptr, ws,
                               need, nullptr) == FLINT_ERR_INVALID_ARG);
      flint_moe_weights bad = w;
      bad.routed.w2 = nullptr;
      EXPECT(flint_moe_forward(ctx, &bad, x, T, out, nullptr, nullptr, ws, need, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      if (fmt == FLINT_W_NVFP4)   // no block scales given
        EXPECT(flint_moe_forward(ctx, &w, x, T, out, nullptr, nullptr, ws, need, nullptr) ==
               FLINT_ERR_INVALID_ARG);
      EXPECT(flint_moe_forward(ctx, &w, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
             FLINT_OK);
      EXPECT(flint_moe_forward_noalloc(ctx, &w, x, -1, out, nullptr, nullptr, nullptr) ==
             FLINT_ERR_INVALID_ARG);
      // the block without gamma, the low-latency path without wo
      EXPECT(flint_moe_block_forward(ctx, &w, nullptr, 1e-6f, x, T, out, nullptr, nullptr, ws, need,
                                     nullptr) == FLINT_ERR_INVALID_ARG);
      EXPECT(flint_moe_lowlat_forward(ctx, &w, nullptr, x, x, fake<const uint16_t>(1u << 21), nullptr,
                                      1e-6f, T, out, nullptr, nullptr, nullptr, ws, need, 1,
                                      nullptr) == FLINT_ERR_INVALID_ARG);
      flint_moe_destroy(ctx);
    }
  }
  EXPECT(flint_moe_forward(nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
         FLINT_ERR_INVALID_ARG);

  // Dense MLP context.
  flint_mlp_ctx* m = nullptr;
  flint_mlp_config mc{2048, 14336, 64};
  EXPECT(flint_mlp_init(&mc, &m) == FLINT_OK && m != nullptr);
  if (m) {
    EXPECT(flint_mlp_workspace_bytes(m, 8) > 0 && flint_mlp_workspace_bytes(m, 0) == 0);
    flint_mlp_ws_layout ml;
    EXPECT(flint_mlp_workspace_layout(m, 8, &ml) == FLINT_OK);
    EXPECT(flint_mlp_forward(m, nullptr, nullptr, nullptr, 1e-6f, nullptr, 8, nullptr, nullptr, 0,
                             nullptr) == FLINT_ERR_INVALID_ARG);
    EXPECT(std::strlen(flint_mlp_last_error(m)) > 0);
    flint_mlp_destroy(m);
  }
  mc.inter = 500;
  m = nullptr;
  EXPECT(flint_mlp_init(&mc, &m) == FLINT_ERR_INVALID_ARG && m == nullptr);

  if (failures) {
    std::fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  std::printf("abi host driver: all checks passed\n");
  return 0;
}
