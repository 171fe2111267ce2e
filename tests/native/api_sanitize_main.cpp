// Drives the host paths of the decode library (hbm_bandwidth_bound_amd/csrc/api.cpp) with the host
// code built under AddressSanitizer and UndefinedBehaviorSanitizer, on a machine without a GPU:
// size queries, argument checks (NULL and misaligned pointers, invalid shapes), the setters and
// queries on a NULL context, status strings, and context creation failing cleanly where no device
// is present. No kernel is launched. Prints "ok" or the first violation. Test code only.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kie.h"
#include "kie_measure.h"

static int fail(const char* what) {
  std::printf("%s\n", what);
  return 1;
}

int main() {
  for (int st = -8; st <= 1; ++st)
    if (!kie_status_string((kie_status)st) || !std::strlen(kie_status_string((kie_status)st)))
      return fail("status string");
  if (!kie_last_error(nullptr)) return fail("last error");

  kie_config cfg;
  std::memset(&cfg, 0, sizeof cfg);
  cfg.n_layers = 2;
  cfg.d_model = 256;
  cfg.n_heads = 4;
  cfg.n_kv_heads = 2;
  cfg.head_dim = 64;
  cfg.ffn_dim = 1024;
  cfg.vocab_size = 4096;
  cfg.rms_eps = 1e-6f;
  cfg.rope_theta = 10000.0f;
  cfg.max_seq_len = 96;
  // sizes depend on the device's compute-unit count: without a device every one is 0, as it is
  // for a NULL or invalid configuration
  if (kie_packed_weight_bytes(&cfg) || kie_kv_cache_bytes(&cfg) || kie_workspace_bytes(&cfg))
    return fail("sizes without a device");
  if (kie_packed_weight_bytes(nullptr) || kie_kv_cache_bytes(nullptr) || kie_workspace_bytes(nullptr))
    return fail("NULL config sizes");
  kie_config bad = cfg;
  bad.n_kv_heads = 3;  // heads not a multiple of the KV heads
  if (kie_kv_cache_bytes(&bad) || kie_packed_weight_bytes(&bad)) return fail("invalid shape sizes");
  if (kie_num_workgroups() > 0) return fail("workgroups without a device");

  // creation: NULL and misaligned buffers are rejected before any device call; with valid-looking
  // pointers the missing device is an error, and *out stays NULL either way
  kie_weights w;
  std::memset(&w, 0, sizeof w);
  kie_ctx* ctx = reinterpret_cast<kie_ctx*>(0x1);
  const uintptr_t base = (uintptr_t)1 << 20;
  void* p = reinterpret_cast<void*>(base);
  if (kie_create(nullptr, &w, p, p, p, nullptr, &ctx) == KIE_OK || ctx) return fail("NULL config");
  if (kie_create(&cfg, nullptr, p, p, p, nullptr, &ctx) == KIE_OK || ctx) return fail("NULL weights");
  if (kie_create(&cfg, &w, p, p, p, nullptr, nullptr) == KIE_OK) return fail("NULL out");
  const uintptr_t mis[4][3] = {
      {base, base + 16, base}, {base, base, base + 64}, {base + 8, base, base}, {0, base, base}};
  for (const auto& m : mis) {
    ctx = reinterpret_cast<kie_ctx*>(0x1);
    if (kie_create(&cfg, &w, reinterpret_cast<void*>(m[0]), reinterpret_cast<void*>(m[1]),
                   reinterpret_cast<void*>(m[2]), nullptr, &ctx) != KIE_ERR_INVALID_ARG ||
        ctx)
      return fail("misaligned or NULL buffer");
  }
  ctx = reinterpret_cast<kie_ctx*>(0x1);
  if (kie_create(&cfg, &w, p, p, p, nullptr, &ctx) == KIE_OK || ctx) return fail("create without a device");
  ctx = reinterpret_cast<kie_ctx*>(0x1);
  if (kie_create_static(&cfg, &w, p, p, nullptr, &ctx) == KIE_OK || ctx)
    return fail("static create without a device");
  if (kie_create(&bad, &w, p, p, p, nullptr, &ctx) == KIE_OK || ctx) return fail("create with an invalid shape");

  // every call on a NULL context is an argument error
  int32_t word = 0;
  if (kie_sync(nullptr) != KIE_ERR_INVALID_ARG || kie_reset(nullptr) != KIE_ERR_INVALID_ARG ||
      kie_set_position(nullptr, 0) != KIE_ERR_INVALID_ARG ||
      kie_set_token_stream(nullptr, &word, 1) != KIE_ERR_INVALID_ARG ||
      kie_set_abort_flag(nullptr, &word) != KIE_ERR_INVALID_ARG || kie_set_skew(nullptr, 1) != KIE_ERR_INVALID_ARG ||
      kie_set_wait_timeout(nullptr, 5) != KIE_ERR_INVALID_ARG)
    return fail("NULL context setters");
  int32_t tok = 0;
  kie_sampling smp{1, 1.0f, 0};
  if (kie_prefill(nullptr, &tok, 1, &tok, nullptr, &smp) == KIE_OK ||
      kie_decode_step(nullptr, &tok, &smp, &tok, nullptr) == KIE_OK ||
      kie_generate(nullptr, &tok, 4, &smp, nullptr, &tok, nullptr) == KIE_OK)
    return fail("NULL context compute calls");
  (void)kie_position(nullptr);
  kie_destroy(nullptr);
  std::printf("ok\n");
  return 0;
}
