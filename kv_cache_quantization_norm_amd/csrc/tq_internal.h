// Internal declarations shared by the host and device halves of libtq.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

// Records a detail message for tq_last_error() and returns `st`.
tq_status fail(tq_status st, const char* fmt, ...);
void clear_error();

constexpr int kVBlock = 32;      // slots per value block
constexpr int kChunk = 32;       // tokens per decode chunk (one wave step)
constexpr int kWaves = 4;        // waves per decode workgroup
constexpr int kMaxGroup = 8;     // query heads handled by one decode workgroup
constexpr int kResidentWorkgroups = 512;  // 256 CUs x 2 decode workgroups

// Format checks shared by all entry points.  `device` additionally requires
// d == 128 and the bit widths the kernels implement.
tq_status check_format(const tq_format* f, bool device);

struct SplitPlan {
  int64_t split_tokens = 0;
  int64_t n_splits = 0;
  int n_head_groups = 0;
  size_t qprep_bytes = 0;    // [L][B][Hq][2][d] fp32
  size_t partial_bytes = 0;  // [L][B][Hq][n_splits][d + 2] fp32
  size_t total_bytes = 0;
};

// Token split and workspace layout of a decode / score call.
SplitPlan plan_decode(int d, int n_layers, int batch, int n_kv_heads, int n_q_heads,
                      int64_t max_seq_len);

}  // namespace tq
