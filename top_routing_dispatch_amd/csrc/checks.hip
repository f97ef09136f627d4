// Host-side checks of the dispatch tables.  With MOE_DEBUG=1 the library
// copies the tables an entry point reads or writes to the host and runs
// these before it goes on (moe_expert_ffn's offsets and gather map,
// moe_combine's row map, moe_permute's and the staged layer's dispatch
// tables); moe_check_dispatch runs the dispatch check on host arrays.
//
// The dispatch tables follow the per-expert batches of "从 Dense FFN 到 MoE"
// §5 (each expert's (token, slot) pairs in row-major order, experts in
// ascending id) with the capacity rule of the "Top-k 路由" page, 容量因子
// (an expert keeps its first C assignments).
#include <stdio.h>

#include <vector>

#include "common.h"
#include "moe.h"

namespace moe {

bool check_group_offsets(const int32_t* off, int G, int max_rows, char* msg, size_t n) {
  if (off[0] < 0) {
    snprintf(msg, n, "offsets[0] = %d is negative", off[0]);
    return false;
  }
  for (int g = 0; g < G; ++g) {
    if (off[g + 1] < off[g]) {
      snprintf(msg, n, "offsets[%d] = %d < offsets[%d] = %d", g + 1, off[g + 1], g, off[g]);
      return false;
    }
  }
  if (off[G] > max_rows) {
    snprintf(msg, n, "offsets[%d] = %d exceeds max_rows = %d", G, off[G], max_rows);
    return false;
  }
  return true;
}

bool check_gather_rows(const int32_t* rows, int n_rows, char* msg, size_t n) {
  for (int r = 0; r < n_rows; ++r) {
    if (rows[r] < 0) {
      snprintf(msg, n, "gather_rows[%d] = %d is negative", r, rows[r]);
      return false;
    }
  }
  return true;
}

bool check_row_map(const int32_t* row_of, int T, int k, int rows_cap, char* msg, size_t n) {
  for (long long i = 0; i < (long long)T * k; ++i) {
    if (row_of[i] < -1 || row_of[i] >= rows_cap) {
      snprintf(msg, n, "row_of[%lld] = %d is outside [-1, %d)", i, row_of[i], rows_cap);
      return false;
    }
  }
  return true;
}

// Recomputes the dispatch of topk_idx (ids outside [0, E) and repeats of an
// id an earlier slot of the token used are skipped) and compares every
// table with it.
bool check_dispatch(const int32_t* idx, const int32_t* counts, const int32_t* offsets, const int32_t* row_of,
                    const int32_t* tor, int T, int k, int E, int capacity, int rows_cap, char* msg, size_t n) {
  std::vector<int32_t> c(E, 0);
  std::vector<int32_t> kept_rank(T * (size_t)k, -1);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      bool ok = e >= 0 && e < E;
      for (int i = 0; ok && i < j; ++i) ok = idx[(size_t)t * k + i] != e;
      if (ok) kept_rank[(size_t)t * k + j] = c[e]++;
    }
  }
  if (offsets[0] != 0) {
    snprintf(msg, n, "offsets[0] = %d, expected 0", offsets[0]);
    return false;
  }
  for (int e = 0; e < E; ++e) {
    if (counts[e] != c[e]) {
      snprintf(msg, n, "counts[%d] = %d, expected %d", e, counts[e], c[e]);
      return false;
    }
    const int kept = c[e] < capacity ? c[e] : capacity;
    if (offsets[e + 1] - offsets[e] != kept) {
      snprintf(msg, n, "offsets[%d] - offsets[%d] = %d, expected %d kept rows", e + 1, e, offsets[e + 1] - offsets[e],
               kept);
      return false;
    }
  }
  if (offsets[E] > rows_cap) {
    snprintf(msg, n, "offsets[%d] = %d exceeds the row bound %d", E, offsets[E], rows_cap);
    return false;
  }
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const size_t i = (size_t)t * k + j;
      const int rk = kept_rank[i];
      const int want = (rk >= 0 && rk < capacity) ? offsets[idx[i]] + rk : -1;
      if (row_of[i] != want) {
        snprintf(msg, n, "row_of[%d][%d] = %d, expected %d", t, j, row_of[i], want);
        return false;
      }
      if (want >= 0 && tor[want] != t) {
        snprintf(msg, n, "token_of_row[%d] = %d, expected %d", want, tor[want], t);
        return false;
      }
    }
  }
  for (int r = offsets[E]; r < rows_cap; ++r) {
    if (tor[r] != -1) {
      snprintf(msg, n, "token_of_row[%d] = %d past the kept rows, expected -1", r, tor[r]);
      return false;
    }
  }
  return true;
}

}  // namespace moe

extern "C" moe_status moe_check_dispatch(const moe_config* cfg, const int32_t* topk_idx, const int32_t* counts,
                                         const int32_t* offsets, const int32_t* row_of,
                                         const int32_t* token_of_row) {
  int32_t capacity = 0, rows_cap = 0;
  const moe_status st = moe_capacity(cfg, &capacity, &rows_cap);
  if (st != MOE_OK) return st;
  const int T = cfg->num_tokens;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (topk_idx == nullptr || row_of == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (rows_cap > 0 && token_of_row == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  char msg[200];
  if (!moe::check_dispatch(topk_idx, counts, offsets, row_of, token_of_row, T, cfg->top_k, cfg->num_experts,
                           capacity, rows_cap, msg, sizeof(msg))) {
    moe::debug_message("moe_check_dispatch", msg);
    return MOE_ERR_DEBUG_CHECK;
  }
  return MOE_OK;
}
