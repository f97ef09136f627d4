// Tuning aids: MOE_* environment variables that force a kernel choice, read
// once per process (and again by moe_reload_tuning), never on a launch path.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "moe.h"

namespace moe {
namespace {

std::once_flag g_tuning_once;
std::mutex g_tuning_mu;
Tuning g_tuning;

int env_int(const char* name) {
  const char* v = getenv(name);
  return (v == nullptr || *v == '\0') ? kUnset : atoi(v);
}

int env_router_path() {
  const char* v = getenv("MOE_ROUTER_PATH");
  if (v == nullptr || *v == '\0') return kUnset;
  if (strcmp(v, "tiled") == 0) return 0;
  if (strcmp(v, "split") == 0) return 1;
  if (strcmp(v, "gemv") == 0) return 2;
  return kUnset;
}

void read_env() {
  Tuning t;
  t.router_kernel = env_int("MOE_ROUTER_KERNEL");
  t.router_path = env_router_path();
  t.gemm_cfg = env_int("MOE_GEMM_CFG");
  t.gemm_cfg_down = env_int("MOE_GEMM_CFG_DOWN");
  t.gemm_ksplit = env_int("MOE_GEMM_KSPLIT");
  t.gemm_shcfg = env_int("MOE_GEMM_SHCFG");
  t.gemm_split = env_int("MOE_GEMM_SPLIT");
  t.gemm_tail = env_int("MOE_GEMM_TAIL");
  t.shared_overlap = env_int("MOE_SHARED_OVERLAP");
  t.shallow_cus = env_int("MOE_SHALLOW_CUS");
  t.tile_gm = env_int("MOE_TILE_GM");
  t.wgrad_tile = env_int("MOE_WGRAD_TILE");
  t.wgrad_swz = env_int("MOE_WGRAD_SWZ");
  t.fused = env_int("MOE_FUSED");
  t.debug = env_int("MOE_DEBUG");
  t.shallow_rows = env_int("MOE_SHALLOW_ROWS");
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  g_tuning = t;
}

}  // namespace

Tuning tuning() {
  std::call_once(g_tuning_once, read_env);
  std::lock_guard<std::mutex> lock(g_tuning_mu);
  return g_tuning;
}

}  // namespace moe

extern "C" moe_status moe_reload_tuning(void) {
  std::call_once(moe::g_tuning_once, [] {});
  moe::read_env();
  return MOE_OK;
}
