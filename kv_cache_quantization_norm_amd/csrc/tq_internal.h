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
constexpr int kDecodeWaves = 8;  // waves per decode workgroup (one workgroup per CU)
constexpr int kDecodeWorkgroups = 256;   // decode workgroups: one per CU of an MI355X
constexpr int kMaxGroup = 8;     // query heads handled by one decode wave
constexpr int kCrossingChunks = 16;   // measured cost of a problem change inside a decode workgroup, in chunks
// The ragged split's padding per problem (its share of a problem change: a
// second piece's merge and pipeline start).  Set apart from kCrossingChunks,
// which decides the static splits: per-workgroup timings on a 16-sequence
// ragged batch of 4 k - 32 k tokens put the change's cost there higher, and
// 16 -> 32 took its decode from 116 to 114 us and its step from 132 to 127 us.
constexpr int kRaggedCrossChunks = 32;
// Ragged split: a problem shorter than the mean range is charged up to
// kContainChunks more, in proportion to how much shorter it is (a range that
// holds a problem whole, with pieces of others on both sides, takes a second
// group: a merge and a pipeline restart in mid-range, measured at about 90
// chunks of time; the weight was tuned on 16-sequence batches of 4 k - 32 k
// tokens).
constexpr int kContainChunks = 160;
constexpr int kRaggedMaxBatch = 1024;  // largest batch whose decode may take the ragged split (its prefix sits in LDS)

// Format checks shared by all entry points.  `device` additionally requires
// d == 128 and the bit widths the kernels implement.
tq_status check_format(const tq_format* f, bool device);

// Work decomposition of a decode / score call.  A problem is one (layer,
// sequence, KV head, head group); its tokens are cut into 32-token chunks,
// chunks_per_problem of them (from max_seq_len, possibly padded with chunks
// that hold no tokens).  The chunks of all problems,
// problem-major, are dealt to n_workgroups workgroups in equal contiguous
// ranges of chunks_per_wg (the last one shorter), so every workgroup has the
// same amount of work; a range may cover the end of one problem and the start
// of the next.  Each (problem, workgroup) piece leaves one partial result in
// its problem's segment slot (at most seg_max slots per problem).
struct SplitPlan {
  int64_t problems = 0;
  int64_t chunks_per_problem = 0;
  int64_t chunks_per_wg = 0;
  int64_t n_workgroups = 0;
  int64_t seg_max = 0;
  int n_head_groups = 0;
  // Ragged split (decided by the kernel from the sequence lengths, batch > 1):
  // the workgroups share the chunks that hold tokens (each problem followed
  // by kRaggedCrossChunks to kRaggedCrossChunks + kContainChunks of padding), in
  // ranges of at least cpw_min chunks, so that a problem (at most cpp_real =
  // ceil(max_len / 32) chunks plus the padding) leaves at most seg_cap
  // pieces; seg_cap >= seg_max is the partial slots per query head in the
  // workspace.
  int64_t cpp_real = 0;
  int64_t cpw_min = 0;
  int64_t seg_cap = 0;
  // Workspace layout, in this order; the counters sit right after the
  // prepared queries, at an offset that does not depend on the work split.
  size_t qprep_bytes = 0;     // [L][B][Hq][2][d] fp32, at offset 0
  size_t counter_offset = 0;  // uint32 [problems] pieces written (in-kernel merge), then [n_layers] append
  size_t counter_bytes = 0;   // counts, then the append wait's give-up flag
  size_t partial_offset = 0;  // [L][B][Hq][seg_cap][d + 2] fp32
  size_t partial_bytes = 0;
  size_t red_offset = 0;      // fp32 [n_workgroups][waves][kMaxGroup][d]: the wave merge of a decode workgroup
  size_t red_bytes = 0;       // (kept in LDS when the tables leave room for it)
  size_t total_bytes = 0;
};

// Work decomposition and workspace layout of a decode / score call.
SplitPlan plan_decode(int d, int n_layers, int batch, int n_kv_heads, int n_q_heads,
                      int64_t max_seq_len, int max_workgroups = kDecodeWorkgroups);

// Decode over a packed cache plus an fp16 tail: each part has its own split;
// the workspace holds the prepared queries twice (for the packed part, then
// plain for the tail), the partials of both parts, the tail's pieces in the
// slots after the packed part's: [L][B][Hq][packed.seg_cap +
// tail.seg_cap][d + 2] fp32, and the packed part's merge counters.
struct TailPlan {
  SplitPlan packed, tail;
  size_t qplain_offset = 0, partial_offset = 0, counter_offset = 0, red_offset = 0, total_bytes = 0;
  int64_t seg_total = 0;
};
TailPlan plan_decode_tail(int d, int n_layers, int batch, int n_kv_heads, int n_q_heads, int64_t max_seq_len,
                          int64_t max_tail_len);

}  // namespace tq
