// Host-only checks of the task-graph builder, validator, simulator and the C ABI's host paths, built
// with AddressSanitizer and UndefinedBehaviorSanitizer (no GPU is touched: contexts are created with
// mk_create_host, and the device launchers are stubs that are never reached). Any memory error or
// undefined behaviour aborts the program with the sanitizer's report; a wrong status exits 1.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mk.h"
#include "../../persistent_megakernel_03_amd/csrc/mk_graph.h"

namespace mk {  // the device-side entry points live in the kernel source, which this build leaves out
hipError_t launch_megakernel(const KernelParams&, int, size_t, hipStream_t, bool) { return hipErrorNotSupported; }
hipError_t megakernel_occupancy(int*, size_t, int, int, int, bool, bool) { return hipErrorNotSupported; }
hipError_t launch_row_scales(const RepackArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_repack_fp8(const RepackArgs&, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_jit_reset(int32_t*, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_repack(const RepackArgs&, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_repack_bias(const uint16_t*, const uint16_t*, const uint16_t*, int, int, int, uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t static_scratch_address(int, void**) { return hipErrorNotSupported; }
hipError_t launch_fill_zero(void*, size_t, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mk

static int failures = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static mk_model_config shape(int L, int d, int hq, int hk, int dh, int f, int v, int seqs, int blocks, int pool) {
  mk_model_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_layers = L; c.d_model = d; c.n_q_heads = hq; c.n_kv_heads = hk; c.head_dim = dh; c.d_ffn = f; c.vocab = v;
  c.rms_eps = 1e-5f; c.rope_theta = 10000.f; c.max_seqs = seqs; c.block_size = 16;
  c.max_blocks_per_seq = blocks; c.num_blocks = pool;
  return c;
}

static void exercise(const mk_model_config& c, int n_cus, int sim_steps, bool corrupt) {
  mk_ctx* ctx = nullptr;
  EXPECT(mk_create_host(&c, n_cus, &ctx) == MK_OK && ctx);
  if (!ctx) return;
  size_t w = 0, kv = 0, s = 0;
  EXPECT(mk_workspace_size(ctx, &w, &kv, &s) == MK_OK && w > 0 && kv > 0 && s > 0);
  mk_graph_info info;
  EXPECT(mk_graph_stats(ctx, &info) == MK_OK && info.n_tasks > 0);
  EXPECT(mk_graph_validate(ctx) == MK_OK);
  if (sim_steps > 0) EXPECT(mk_graph_simulate(ctx, 7, sim_steps) == MK_OK);
  // device calls on a host context are refused without touching a device
  EXPECT(mk_decode_step(ctx, (const int32_t*)16, 1, (int32_t*)16, nullptr) == MK_ERR_STATE);
  EXPECT(mk_decode_n(ctx, (const int32_t*)16, 1, 4, (int32_t*)16, nullptr) == MK_ERR_STATE);
  EXPECT(mk_sync_check(ctx, nullptr) == MK_ERR_STATE);
  mk_destroy(ctx);
  if (!corrupt) return;
  for (int kind = 1; kind <= 7; ++kind) {
    mk_ctx* b = nullptr;
    if (mk_create_host(&c, n_cus, &b) != MK_OK) { ++failures; continue; }
    if (mk_graph_corrupt(b, kind) == MK_OK) {
      if (kind == 6) {
        (void)mk_graph_validate(b);
        for (uint64_t seed = 0; seed < 4; ++seed) (void)mk_graph_simulate(b, seed, 1);
      } else {
        EXPECT(mk_graph_validate(b) == MK_ERR_SHAPE);
      }
    }
    mk_destroy(b);
  }
}

int main() {
  // the tiny decoder on many and on few CUs, a GQA 7:1 odd shape, the 8B shape (no simulation: large)
  exercise(shape(2, 256, 4, 2, 64, 688, 4096, 1, 3, 3), 256, 3, true);
  exercise(shape(2, 256, 4, 2, 64, 688, 4096, 1, 3, 3), 7, 3, true);
  exercise(shape(2, 448, 7, 1, 64, 1216, 1000, 1, 5, 5), 19, 2, true);
  exercise(shape(32, 4096, 32, 8, 128, 14336, 128256, 1, 35, 35), 256, 0, false);
  exercise(shape(32, 4096, 32, 8, 128, 14336, 128256, 1, 2052, 2052), 256, 0, false);
  // batched: tiny with 4 sequences, the mid shape with 16 (column splits), 8B with 16
  exercise(shape(2, 256, 4, 2, 64, 688, 4096, 4, 4, 16), 256, 2, true);
  exercise(shape(2, 2048, 16, 4, 128, 5632, 16384, 16, 4, 64), 256, 1, true);
  exercise(shape(32, 4096, 32, 8, 128, 14336, 128256, 16, 377, 3407), 256, 0, false);
  // bad configurations and arguments are refused, with no context leaked
  mk_ctx* ctx = nullptr;
  mk_model_config bad = shape(2, 250, 4, 2, 64, 688, 4096, 1, 3, 3);
  EXPECT(mk_create_host(&bad, 256, &ctx) == MK_ERR_SHAPE && ctx == nullptr);
  bad = shape(2, 256, 4, 2, 96, 688, 4096, 1, 3, 3);
  EXPECT(mk_create_host(&bad, 256, &ctx) == MK_ERR_SHAPE);
  bad = shape(2, 256, 4, 2, 64, 688, 4096, 17, 3, 3);
  EXPECT(mk_create_host(&bad, 256, &ctx) == MK_ERR_SHAPE);
  bad = shape(2, 256, 4, 2, 64, 688, 4096, 1, 3, 3);
  EXPECT(mk_create_host(&bad, 0, &ctx) == MK_ERR_SHAPE);
  EXPECT(mk_create_host(nullptr, 256, &ctx) == MK_ERR_INVALID_ARG);
  EXPECT(mk_graph_validate(nullptr) == MK_ERR_INVALID_ARG);
  EXPECT(mk_graph_stats(nullptr, nullptr) == MK_ERR_INVALID_ARG);
  EXPECT(std::strlen(mk_last_error()) > 0);
  EXPECT(std::strcmp(mk_status_str(MK_ERR_DEVICE_TIMEOUT), "MK_ERR_DEVICE_TIMEOUT") == 0);
  mk_destroy(nullptr);
  std::printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
