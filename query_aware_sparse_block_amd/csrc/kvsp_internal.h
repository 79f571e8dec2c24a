// Kernel argument blocks and launchers shared between the kvsp kernels and the
// C entry points. Internal header: not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsp.h"

namespace kvsp {

struct SummaryArgs {
  const void* k_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* summaries;
  int32_t B, Hkv, P, max_blocks;
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* block_table;
  const int32_t* positions;
  void* k_pool;
  void* v_pool;
  float* summaries;
  int32_t B, Hkv, P, max_blocks, num_phys;
};

struct ScoreArgs {
  const void* q;
  const float* summaries;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* scores;  // [B][max_blocks]
  int32_t B, Hq, Hkv, D, P, max_blocks;
  int32_t blocks_per_wave;
  int32_t stream_rows;  // 1: read summary rows with non-temporal loads
  int32_t top_k, keep_num, keep_den, keep_floor, recent_window, gamma_num, gamma_den;
};

struct TopkArgs {
  const float* scores;
  const int32_t* context_lens;
  int32_t* selected;
  int32_t* num_selected;
  int32_t* spans;
  int32_t* num_spans;
  int32_t* use_dense;
  int32_t B, P, max_blocks;
  int32_t top_k, keep_num, keep_den, keep_floor, recent_window, gamma_num, gamma_den;
};

// Split-KV decode. The attended token sequence of sequence b (selected blocks
// then the window, or every block when dense) is cut into at most `max_chunks`
// chunks of whole sub-tiles; each (sequence, KV head, head group, chunk) is one
// work item for one workgroup. Partials live at slot
//   ((b * Hkv + g) * n_head_groups + hg) * max_chunks + c,
// and counters[(b * Hkv + g) * n_head_groups + hg] counts finished chunks.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* selected;      // NULL when every sequence is dense or spans are given
  const int32_t* num_selected;  // NULL when every sequence is dense or spans are given
  const int32_t* spans;         // [B][max_blocks + 1][2]; NULL: use `selected`
  const int32_t* num_spans;     // [B]; with `spans`
  const int32_t* use_dense;     // may be NULL
  float* out;
  float* lse;                   // may be NULL
  float* part_acc;              // [slots][GP][D]
  float* part_ml;               // [slots][GP][2]
  int32_t* counters;            // [B * Hkv * n_head_groups], zero between calls
  int32_t B, Hq, Hkv, D, P, max_blocks;
  int32_t recent_window;
  int32_t all_dense;            // 1: ignore selection, attend every token
  int32_t n_head_groups;        // ceil(G / GP)
  int32_t max_chunks;
  int32_t total_items;          // B * Hkv * n_head_groups * max_chunks
  int32_t xcd_share;            // 1: the head groups of a KV head's chunk share an XCD
  float scale_log2;             // softmax scale * log2(e)
};

// DKV decode over compressed blocks and the exact window, one launch. Work
// item (chunk slot c, pair = b * Hkv + g), numbered item = c * B * Hkv + pair,
// with S = n_chunks + n_wchunks slots per pair. Slot c < n_chunks takes
// selected blocks [c * per, min(k, (c + 1) * per)), per = ceil(k / n_chunks);
// slot n_chunks + w takes 64-token window groups [w * wper, ...), wper =
// ceil(groups / n_wchunks). Active chunks are numbered compressed first;
// partials live at slot pair * S + that number; counters[pair] counts
// finished chunks.
struct DkvDecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const char* records;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* selected;
  const int32_t* num_selected;
  float* out;
  float* lse;                   // may be NULL
  float* part_acc;              // [slots][16][D]
  float* part_ml;               // [slots][16][2]
  int32_t* counters;            // [B * Hkv], zero between calls
  int64_t rec_bytes;
  int32_t off_basis, off_coef, off_rk, off_rv, off_ridx;
  int32_t B, Hq, Hkv, P, max_blocks, recent_window, n_resid, n_chunks, n_wchunks;
  float scale_log2;
};
// DKV codec: one work item per (sequence, candidate block, KV head).
// power_iters > 0: exactly that many subspace-iteration rounds; 0: rounds
// chosen per block from the Ritz values after the first rounds.
struct DkvCompressArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  char* records;
  int64_t rec_bytes;
  int32_t off_basis, off_coef, off_rk, off_rv, off_ridx, off_rounds;
  int32_t B, Hkv, P, max_blocks, num_phys, recent_window, n_resid, power_iters;
};
hipError_t launch_dkv_decode(const DkvDecodeArgs& a, int dtype, int D, hipStream_t stream);
hipError_t launch_dkv_compress(const DkvCompressArgs& a, int dtype, int D, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int dtype, int D, hipStream_t stream);
hipError_t launch_build_summaries(const SummaryArgs& a, int dtype, int D, hipStream_t stream);
hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
// Scores and Top-k in one launch (when fused_select_supported for the table
// length and the scoring workgroups of the whole batch, score_workgroups);
// counters: [B] ints, zero between calls.
int64_t score_workgroups(const ScoreArgs& sa);
bool fused_select_supported(int max_blocks, int64_t workgroups);
hipError_t launch_score_select(const ScoreArgs& sa, const TopkArgs& ta, int32_t* counters,
                               int dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int group_pad, int num_wgs,
                         hipStream_t stream);
// The same for a K pool in host memory (row-major K loads; kvsp_decode_host.hip).
hipError_t launch_decode_host(const DecodeArgs& a, int dtype, int group_pad, int num_wgs,
                              hipStream_t stream);

// Host-side sizing shared by the entry points and kvsp_workspace_bytes.
int decode_group_pad(const kvsp_layout& l);  // GP: heads per work item (1, 2, 4, 8 or 16)
int decode_max_chunks(const kvsp_layout& l);
int decode_chunk_quantum(int dtype, int D);  // tokens per chunk unit
struct ScoreShape {
  int lg, vpl;  // lanes that share one summary row, 16-byte vectors per lane
};
ScoreShape score_shape(int Hkv, int D);

}  // namespace kvsp
