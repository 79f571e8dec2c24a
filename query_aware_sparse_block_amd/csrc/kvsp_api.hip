// C entry points of libkvsp: argument checks, workspace layout and launch
// geometry. Every check runs on the host before anything is enqueued; no
// entry point allocates, synchronises or copies to the host.

#include <stddef.h>
#include <algorithm>
#include <cmath>
#include <mutex>
#include <stdint.h>

#include "kvsp.h"
#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {
namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxBlocksPerSeq = 16384;
// Bounds that keep every work-item count and per-head product in int32.
constexpr int kMaxBatch = 65536;
constexpr int kMaxQHeads = 1024;
constexpr int kMaxSummaryRow = 7168;   // Hkv * D: the score kernel stages it in LDS as double
// Workgroup items per decode launch (about one per resident workgroup) and the
// cap on launched workgroups; items beyond it are taken in grid-stride order.
#ifndef KVSP_DECODE_TARGET_ITEMS
#define KVSP_DECODE_TARGET_ITEMS 256
#endif
#ifndef KVSP_DECODE_MAX_WORKGROUPS
#define KVSP_DECODE_MAX_WORKGROUPS 2048
#endif
constexpr int kDecodeTargetItems = KVSP_DECODE_TARGET_ITEMS;
// The merge gives each chunk of a group one lane of a wavefront, and keeps a
// weight per (chunk, head) plus (M, Lsum) per head in the kernel's LDS (the
// 3 * GP * D floats of its wave-merge buffer): at most 64 chunks.
constexpr int kDecodeMaxChunks = 64;
// Heads per work item: the group's query heads padded to a power of two (at
// most 16). With few (sequence, KV head) pairs the heads are split into
// smaller groups, down to KVSP_DECODE_MIN_GP, until there are
// KVSP_DECODE_SPLIT_GROUPS groups: each group then merges its own partials,
// at the price of reading the KV head once per group.
#ifndef KVSP_DECODE_SPLIT_GROUPS
#define KVSP_DECODE_SPLIT_GROUPS 8
#endif
#ifndef KVSP_DECODE_MIN_GP
#define KVSP_DECODE_MIN_GP 4
#endif
// Scoring workgroups a launch aims for (a sequence's candidates are split
// into whole waves' worth of blocks; short tables keep one pass per wave).
// Measured on the serving shape with the separate Top-k launch: 1024 (four
// workgroups per CU) scores faster than 512, 768 or 1536.
#ifndef KVSP_SCORE_TARGET_WORKGROUPS
#define KVSP_SCORE_TARGET_WORKGROUPS 1024
#endif
constexpr int kScoreTargetWorkgroups = KVSP_SCORE_TARGET_WORKGROUPS;
// Calls reading more summary bytes than this use non-temporal loads for them:
// measured faster for the 128 MiB of the serving shape, slower for the 8 MiB
// of the OPT-like batch, which can stay in the 256 MB Infinity Cache.
constexpr int64_t kScoreStreamBytes = int64_t(64) << 20;
constexpr int kDecodeMaxWorkgroups = KVSP_DECODE_MAX_WORKGROUPS;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

kvsp_status check_layout(const kvsp_layout* l) {
  if (l == nullptr) return KVSP_ERR_INVALID_ARG;
  if (l->batch < 1 || l->num_q_heads < 1 || l->num_kv_heads < 1 || l->num_phys_blocks < 1 ||
      l->max_blocks_per_seq < 1)
    return KVSP_ERR_INVALID_ARG;
  if (l->num_q_heads % l->num_kv_heads != 0) return KVSP_ERR_INVALID_ARG;
  if (l->batch > kMaxBatch || l->num_q_heads > kMaxQHeads) return KVSP_ERR_UNSUPPORTED;
  if (l->head_dim != 64 && l->head_dim != 128) return KVSP_ERR_UNSUPPORTED;
  if (!pow2(l->block_size) || l->block_size < 16 || l->block_size > 256) return KVSP_ERR_UNSUPPORTED;
  if (l->dtype != KVSP_F32 && l->dtype != KVSP_F16 && l->dtype != KVSP_BF16) return KVSP_ERR_UNSUPPORTED;
  if (l->max_blocks_per_seq > kMaxBlocksPerSeq) return KVSP_ERR_UNSUPPORTED;
  if (l->num_kv_heads * l->head_dim > kMaxSummaryRow) return KVSP_ERR_UNSUPPORTED;
  return KVSP_OK;
}

kvsp_status check_params(const kvsp_select_params* p) {
  if (p == nullptr) return KVSP_ERR_INVALID_ARG;
  if (p->top_k < 0 || p->keep_num < 0 || p->keep_den <= 0 || p->keep_floor < 0 ||
      p->recent_window < 0 || p->gamma_num < 0 || p->gamma_den <= 0)
    return KVSP_ERR_INVALID_ARG;
  // With neither a floor nor a window the attended set could be empty.
  if (p->keep_floor == 0 && p->recent_window == 0) return KVSP_ERR_INVALID_ARG;
  return KVSP_OK;
}

struct WorkspaceLayout {
  size_t counters, select_counters, part_acc, part_ml, scores, total;
};

struct DecodeGeometry {
  int gp, n_head_groups, max_chunks, total_items, num_wgs;
};

DecodeGeometry decode_geometry(const kvsp_layout& l) {
  DecodeGeometry d;
  const int G = l.num_q_heads / l.num_kv_heads;
  d.gp = decode_group_pad(l);
  d.n_head_groups = (G + d.gp - 1) / d.gp;
  d.max_chunks = decode_max_chunks(l);
  d.total_items = l.batch * l.num_kv_heads * d.n_head_groups * d.max_chunks;
  d.num_wgs = d.total_items < kDecodeMaxWorkgroups ? d.total_items : kDecodeMaxWorkgroups;
  return d;
}

WorkspaceLayout workspace_layout(const kvsp_layout& l) {
  const DecodeGeometry d = decode_geometry(l);
  const size_t slots = static_cast<size_t>(d.total_items);
  WorkspaceLayout w;
  size_t off = 0;
  w.counters = off;
  off += align_up(static_cast<size_t>(l.batch) * l.num_kv_heads * d.n_head_groups * sizeof(int32_t));
  w.select_counters = off;
  off += align_up(static_cast<size_t>(l.batch) * sizeof(int32_t));
  w.part_acc = off;
  off += align_up(slots * d.gp * l.head_dim * sizeof(float));
  w.part_ml = off;
  off += align_up(slots * d.gp * 2 * sizeof(float));
  w.scores = off;
  off += align_up(static_cast<size_t>(l.batch) * l.max_blocks_per_seq * sizeof(float));
  w.total = off;
  return w;
}

kvsp_status from_hip(hipError_t e) { return e == hipSuccess ? KVSP_OK : KVSP_ERR_HIP; }

// True if p lies in host memory mapped for the device (a pool kept in host
// RAM): there the decode reads K row-major, in larger PCIe requests.
// Device memory, and anything HIP does not know, count as device memory.
bool in_host_memory(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // consumed here, so the launch check does not report it
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

// Host checks shared by every decode entry point (no HIP call).
kvsp_status check_decode(const kvsp_layout* layout, const kvsp_select_params* params, bool all_dense,
                         const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_table, const int32_t* context_lens,
                         const int32_t* spans, const int32_t* num_spans,
                         const int32_t* selected, const int32_t* num_selected, const float* out) {
  kvsp_status st = check_layout(layout);
  if (st != KVSP_OK) return st;
  if (!all_dense && (st = check_params(params)) != KVSP_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out)
    return KVSP_ERR_INVALID_ARG;
  if (!all_dense) {
    // exactly one form of the kept blocks: the span list or the selected list
    const bool by_spans = spans != nullptr || num_spans != nullptr;
    const bool by_list = selected != nullptr || num_selected != nullptr;
    if (by_spans == by_list) return KVSP_ERR_INVALID_ARG;
    if (by_spans && (!spans || !num_spans)) return KVSP_ERR_INVALID_ARG;
    if (by_list && (!selected || !num_selected)) return KVSP_ERR_INVALID_ARG;
  }
  return KVSP_OK;
}

// Where a decode keeps its completion counters and split-KV partials.
struct DecodeScratch {
  int32_t* counters;
  float* part_acc;
  float* part_ml;
};

DecodeScratch workspace_scratch(const kvsp_layout& l, void* workspace) {
  const WorkspaceLayout wl = workspace_layout(l);
  char* base = static_cast<char*>(workspace);
  return {reinterpret_cast<int32_t*>(base + wl.counters), reinterpret_cast<float*>(base + wl.part_acc),
          reinterpret_cast<float*>(base + wl.part_ml)};
}

// Launches the decode of checked arguments into `scr`.
kvsp_status launch_checked_decode(const kvsp_layout& l, const kvsp_select_params* params,
                                  bool all_dense, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_table,
                                  const int32_t* context_lens, const int32_t* spans,
                                  const int32_t* num_spans, const int32_t* selected,
                                  const int32_t* num_selected, const int32_t* use_dense,
                                  float scale, float* out, float* lse, const DecodeScratch& scr,
                                  hipStream_t stream) {
  const DecodeGeometry g = decode_geometry(l);
  DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.selected = all_dense ? nullptr : selected;
  a.num_selected = all_dense ? nullptr : num_selected;
  a.spans = all_dense ? nullptr : spans;
  a.num_spans = all_dense ? nullptr : num_spans;
  a.use_dense = all_dense ? nullptr : use_dense;
  a.out = out;
  a.lse = lse;
  a.part_acc = scr.part_acc;
  a.part_ml = scr.part_ml;
  a.counters = scr.counters;
  a.B = l.batch;
  a.Hq = l.num_q_heads;
  a.Hkv = l.num_kv_heads;
  a.D = l.head_dim;
  a.P = l.block_size;
  a.max_blocks = l.max_blocks_per_seq;
  a.recent_window = all_dense ? 0 : params->recent_window;
  a.all_dense = all_dense ? 1 : 0;
  a.n_head_groups = g.n_head_groups;
  a.max_chunks = g.max_chunks;
  a.total_items = g.total_items;
  // Several head groups per KV head re-read its tiles: keep each chunk's
  // groups on one XCD (the renumbering needs whole rounds of 8 XCDs x groups
  // and a grid that is a multiple of 8).
  a.xcd_share = (g.n_head_groups > 1 && g.total_items % (8 * g.n_head_groups) == 0 &&
                 g.num_wgs % 8 == 0) ? 1 : 0;
  const float s = scale > 0.f ? scale : 1.0f / __builtin_sqrtf(static_cast<float>(l.head_dim));
  a.scale_log2 = s * 1.4426950408889634f;
  if (in_host_memory(k_pool)) return from_hip(launch_decode_host(a, l.dtype, g.gp, g.num_wgs, stream));
  return from_hip(launch_decode(a, l.dtype, g.gp, g.num_wgs, stream));
}

kvsp_status run_decode(const kvsp_layout* layout, const kvsp_select_params* params, bool all_dense,
                       const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* context_lens,
                       const int32_t* spans, const int32_t* num_spans,
                       const int32_t* selected, const int32_t* num_selected,
                       const int32_t* use_dense, float scale, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const kvsp_status st = check_decode(layout, params, all_dense, q, k_pool, v_pool, block_table,
                                      context_lens, spans, num_spans, selected, num_selected, out);
  if (st != KVSP_OK) return st;
  const kvsp_layout& l = *layout;
  if (workspace == nullptr || workspace_bytes < workspace_layout(l).total) return KVSP_ERR_WORKSPACE;
  return launch_checked_decode(l, params, all_dense, q, k_pool, v_pool, block_table, context_lens,
                               spans, num_spans, selected, num_selected, use_dense, scale, out,
                               lse, workspace_scratch(l, workspace), stream);
}

// ---- the decode for callers that cannot allocate --------------------------------
// Its counters and partials live in `scratch`, a file-scope device array (one
// copy per device, held until the process ends). The completion counters
// have a fixed region at its start, so a later call's counters never overlap
// an earlier call's partials; the kernels leave them at zero after every
// call, and a fill kernel zeroes them once per device at set-up. Partials
// follow at a fixed offset; they are needed only when a group is split into
// several chunks.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr size_t kStaticCounterBytes = size_t(64) << 10;  // 16384 groups
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct DeviceScratch {
  char* ptr = nullptr;   // the device address of `scratch` on this device
  bool cleared = false;  // counters zeroed by an eager (not captured) fill
};
std::mutex g_scratch_mutex;
DeviceScratch g_scratch[kMaxDevices];

__global__ void zero_words(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Bytes of `scratch` a decode of this layout uses, or 0 if it does not fit.
size_t static_decode_bytes(const kvsp_layout& l) {
  const DecodeGeometry g = decode_geometry(l);
  const size_t groups = static_cast<size_t>(l.batch) * l.num_kv_heads * g.n_head_groups;
  if (groups * sizeof(int32_t) > kStaticCounterBytes) return 0;
  size_t need = kStaticCounterBytes;
  if (g.max_chunks > 1) {
    const size_t slots = static_cast<size_t>(g.total_items);
    need += align_up(slots * g.gp * l.head_dim * sizeof(float)) + align_up(slots * g.gp * 2 * sizeof(float));
  }
  return need <= kStaticScratchBytes ? need : 0;
}

// The current device's copy of `scratch`, its counters zeroed on `stream`
// ahead of first use.
kvsp_status static_scratch(const kvsp_layout& l, hipStream_t stream, DecodeScratch* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVSP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KVSP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  DeviceScratch& d = g_scratch[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return KVSP_ERR_HIP;
    d.ptr = static_cast<char*>(p);
  }
  if (!d.cleared) {
    // A fill kernel, not a memset, so that a captured first call records a
    // kernel node; only an eager fill counts as done.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return KVSP_ERR_HIP;
    constexpr int words = static_cast<int>(kStaticCounterBytes / sizeof(int32_t));
    hipLaunchKernelGGL(zero_words, dim3(words / 256), dim3(256), 0, stream,
                       reinterpret_cast<int32_t*>(d.ptr), words);
    if (hipGetLastError() != hipSuccess) return KVSP_ERR_HIP;
    if (cap == hipStreamCaptureStatusNone) d.cleared = true;
  }
  const DecodeGeometry g = decode_geometry(l);
  const size_t slots = static_cast<size_t>(g.total_items);
  char* acc = d.ptr + kStaticCounterBytes;
  out->counters = reinterpret_cast<int32_t*>(d.ptr);
  out->part_acc = reinterpret_cast<float*>(acc);
  out->part_ml = reinterpret_cast<float*>(acc + align_up(slots * g.gp * l.head_dim * sizeof(float)));
  return KVSP_OK;
}

// ---- DKV variant ------------------------------------------------------------------

constexpr int kDkvRank = 32;
constexpr int kDkvMaxResid = 64;
constexpr int kDkvMaxHeads = 16;      // query heads per KV head (MFMA columns)
constexpr int kDkvTargetItems = 256;  // decode work items a launch aims for
constexpr int kDkvMaxChunks = 32;     // compressed-block chunks per (sequence, KV head)
constexpr int kDkvMaxWindowChunks = 32;  // window chunks per (sequence, KV head)

struct DkvRecordLayout {
  int32_t off_basis, off_coef, off_rk, off_rv, off_ridx, off_rounds;
  size_t bytes;
};

size_t align_to(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elem_bytes(int dtype) { return dtype == KVSP_F32 ? 4 : 2; }

DkvRecordLayout dkv_record_layout(const kvsp_layout& l, int n_resid) {
  const size_t D = static_cast<size_t>(l.head_dim), P = static_cast<size_t>(l.block_size);
  const size_t E = static_cast<size_t>(elem_bytes(l.dtype));
  DkvRecordLayout r;
  size_t off = align_to(2 * D * E, 16);
  r.off_basis = static_cast<int32_t>(off);
  off += kDkvRank * 2 * D * 4;
  r.off_coef = static_cast<int32_t>(off);
  off += P * kDkvRank * 4;
  r.off_rk = static_cast<int32_t>(off);
  off += static_cast<size_t>(n_resid) * D * E;
  r.off_rv = static_cast<int32_t>(off);
  off += static_cast<size_t>(n_resid) * D * E;
  r.off_ridx = static_cast<int32_t>(off);
  off += static_cast<size_t>(n_resid) * 4;
  r.off_rounds = static_cast<int32_t>(off);
  off += 4;
  r.bytes = align_to(off, 256);
  return r;
}

kvsp_status check_dkv(const kvsp_layout* l, const kvsp_dkv_params* p) {
  kvsp_status st = check_layout(l);
  if (st != KVSP_OK) return st;
  if (p == nullptr) return KVSP_ERR_INVALID_ARG;
  if (p->rank != kDkvRank) return KVSP_ERR_UNSUPPORTED;
  if (p->n_resid < 0 || p->power_iters < 0 || p->power_iters > 1000) return KVSP_ERR_INVALID_ARG;
  if (l->block_size < 64) return KVSP_ERR_UNSUPPORTED;
  if (p->n_resid > kDkvMaxResid || p->n_resid > l->block_size) return KVSP_ERR_UNSUPPORTED;
  if (l->num_q_heads / l->num_kv_heads > kDkvMaxHeads) return KVSP_ERR_UNSUPPORTED;
  return KVSP_OK;
}

int dkv_chunks(const kvsp_layout& l) {
  const int64_t pairs = static_cast<int64_t>(l.batch) * l.num_kv_heads;
  int nc = 1;
  while (pairs * nc < kDkvTargetItems && nc < kDkvMaxChunks && nc < l.max_blocks_per_seq) nc *= 2;
  return nc;
}

// Window chunks: the window holds at most W + P - 1 tokens (and no more than
// the table), cut into 64-token groups; at most kDkvMaxWindowChunks chunks.
int dkv_window_chunks(const kvsp_layout& l, int32_t recent_window) {
  const int64_t cap = static_cast<int64_t>(l.max_blocks_per_seq) * l.block_size;
  const int64_t tokens = std::min<int64_t>(static_cast<int64_t>(recent_window) + l.block_size - 1, cap);
  const int64_t groups = (tokens + 63) / 64;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(groups, kDkvMaxWindowChunks)));
}

struct DkvWorkspace {
  size_t counters, part_acc, part_ml, total;
};

// Sized for the most window chunks, so it does not depend on the window.
DkvWorkspace dkv_workspace(const kvsp_layout& l) {
  DkvWorkspace w;
  const size_t slots = static_cast<size_t>(l.batch) * l.num_kv_heads *
                       (dkv_chunks(l) + kDkvMaxWindowChunks);
  size_t off = 0;
  w.counters = off;
  off += align_up(static_cast<size_t>(l.batch) * l.num_kv_heads * sizeof(int32_t));
  w.part_acc = off;
  off += align_up(slots * kDkvMaxHeads * l.head_dim * sizeof(float));
  w.part_ml = off;
  off += align_up(slots * kDkvMaxHeads * 2 * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace

int decode_group_pad(const kvsp_layout& l) {
  const int G = l.num_q_heads / l.num_kv_heads;
  const int gp0 = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
  int gp = gp0;
  const int64_t pairs = static_cast<int64_t>(l.batch) * l.num_kv_heads;
  while (gp > KVSP_DECODE_MIN_GP && pairs * ((G + gp - 1) / gp) < KVSP_DECODE_SPLIT_GROUPS) gp /= 2;
  // Once split, halve again while that removes padded head slots (6 heads in
  // items of 4 pad 2 slots, in items of 2 none): measured 14.5 -> 12.8 us on
  // the Qwen-like shape, while 16 heads stay in items of 4 (2 was slower).
  if (gp < gp0) {
    auto slots = [G](int g) { return (G + g - 1) / g * g; };
    while (gp > 2 && slots(gp / 2) < slots(gp)) gp /= 2;
  }
  return gp;
}

// Chunks per (sequence, KV head, head group): enough workgroup items to
// occupy the chip (about kDecodeTargetItems), never more than the longest
// possible context has chunk quanta.
int decode_max_chunks(const kvsp_layout& l) {
  const int G = l.num_q_heads / l.num_kv_heads;
  const int gp = decode_group_pad(l);
  const int64_t groups = static_cast<int64_t>(l.batch) * l.num_kv_heads * ((G + gp - 1) / gp);
  const int quantum = decode_chunk_quantum(l.dtype, l.head_dim);
  const int64_t max_sub = (static_cast<int64_t>(l.max_blocks_per_seq) * l.block_size + quantum - 1) / quantum;
  int64_t mc = 1;
  while (groups * mc < kDecodeTargetItems && mc < max_sub && mc < kDecodeMaxChunks) mc *= 2;
  return static_cast<int>(mc);
}

}  // namespace kvsp

using namespace kvsp;

extern "C" {

int32_t kvsp_abi_version(void) { return KVSP_ABI_VERSION; }

const char* kvsp_status_string(kvsp_status s) {
  switch (s) {
    case KVSP_OK: return "ok";
    case KVSP_ERR_INVALID_ARG: return "invalid argument";
    case KVSP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case KVSP_ERR_WORKSPACE: return "workspace missing or too small";
    case KVSP_ERR_HIP: return "HIP launch failed";
    case KVSP_ERR_TOO_LARGE: return "layout needs more than the static scratch of kvsp_sparse_decode_noalloc";
  }
  return "unknown status";
}

size_t kvsp_workspace_bytes(const kvsp_layout* layout, const kvsp_select_params* params) {
  (void)params;
  if (check_layout(layout) != KVSP_OK) return 0;
  return workspace_layout(*layout).total;
}

// SparPR, "Dynamic budget control": the copy price of a block (its bytes over
// the host-to-device bandwidth, twice for K and V) against its recompute price
// (the K and V projections of its hidden states), the ratio read as the keep
// ratio (capped at 1) in units of 1/keep_den, rounded up.
kvsp_status kvsp_budget_keep_ratio(const kvsp_layout* layout, const kvsp_budget_model* model,
                                   int32_t keep_den, double* copy_s, double* recompute_s,
                                   int32_t* keep_num) {
  const kvsp_status st = check_layout(layout);
  if (st != KVSP_OK) return st;
  if (model == nullptr || keep_num == nullptr || keep_den <= 0) return KVSP_ERR_INVALID_ARG;
  const double bandwidth = model->h2d_bytes_per_s;
  const double throughput = model->proj_flops_per_s;
  if (!std::isfinite(bandwidth) || !(bandwidth > 0.0) || !std::isfinite(throughput) ||
      !(throughput > 0.0) || model->hidden <= 0)
    return KVSP_ERR_INVALID_ARG;
  const double tokens = layout->block_size;
  const double kv_width = static_cast<double>(layout->num_kv_heads) * layout->head_dim;
  const double copy = 2.0 * tokens * kv_width * elem_bytes(layout->dtype) / bandwidth;
  const double recompute = 4.0 * tokens * static_cast<double>(model->hidden) * kv_width / throughput;
  const double ratio = std::min(1.0, recompute / copy);
  const double units = std::ceil(ratio * keep_den);
  int32_t num = keep_den;
  if (units < static_cast<double>(keep_den)) num = units < 1.0 ? 1 : static_cast<int32_t>(units);
  if (copy_s != nullptr) *copy_s = copy;
  if (recompute_s != nullptr) *recompute_s = recompute;
  *keep_num = num;
  return KVSP_OK;
}

kvsp_status kvsp_append_kv(const kvsp_layout* layout, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* positions, void* k_pool,
                           void* v_pool, float* summaries, hipStream_t stream) {
  kvsp_status st = check_layout(layout);
  if (st != KVSP_OK) return st;
  if (!k_new || !v_new || !block_table || !positions || !k_pool || !v_pool || !summaries)
    return KVSP_ERR_INVALID_ARG;
  const kvsp_layout& l = *layout;
  AppendArgs a{k_new, v_new, block_table, positions, k_pool, v_pool, summaries, l.batch,
               l.num_kv_heads, l.block_size, l.max_blocks_per_seq, l.num_phys_blocks};
  return from_hip(launch_append(a, l.dtype, l.head_dim, stream));
}

kvsp_status kvsp_build_summaries(const kvsp_layout* layout, const void* k_pool,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 float* summaries, hipStream_t stream) {
  kvsp_status st = check_layout(layout);
  if (st != KVSP_OK) return st;
  if (!k_pool || !block_table || !context_lens || !summaries) return KVSP_ERR_INVALID_ARG;
  const kvsp_layout& l = *layout;
  SummaryArgs a{k_pool, block_table, context_lens, summaries, l.batch, l.num_kv_heads,
                l.block_size, l.max_blocks_per_seq};
  return from_hip(launch_build_summaries(a, l.dtype, l.head_dim, stream));
}

kvsp_status kvsp_score_topk(const kvsp_layout* layout, const kvsp_select_params* params,
                            const void* q, const float* summaries, const int32_t* block_table,
                            const int32_t* context_lens, float* scores, int32_t* selected,
                            int32_t* num_selected, int32_t* spans, int32_t* num_spans,
                            int32_t* use_dense, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  kvsp_status st = check_layout(layout);
  if (st != KVSP_OK) return st;
  if ((st = check_params(params)) != KVSP_OK) return st;
  if (!q || !summaries || !block_table || !context_lens || !selected || !num_selected || !spans ||
      !num_spans || !use_dense)
    return KVSP_ERR_INVALID_ARG;
  const kvsp_layout& l = *layout;
  const kvsp_select_params& p = *params;
  const WorkspaceLayout wl = workspace_layout(l);
  if (workspace == nullptr || workspace_bytes < wl.total) return KVSP_ERR_WORKSPACE;
  if (scores == nullptr) scores = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.scores);
  ScoreArgs sa;
  sa.q = q;
  sa.summaries = summaries;
  sa.block_table = block_table;
  sa.context_lens = context_lens;
  sa.scores = scores;
  sa.B = l.batch;
  sa.Hq = l.num_q_heads;
  sa.Hkv = l.num_kv_heads;
  sa.D = l.head_dim;
  sa.P = l.block_size;
  sa.max_blocks = l.max_blocks_per_seq;
  // About kScoreTargetWorkgroups workgroups of four waves over all candidates.
  const int64_t total_blocks = static_cast<int64_t>(l.batch) * l.max_blocks_per_seq;
  int64_t bpw = (total_blocks + 4 * kScoreTargetWorkgroups - 1) / (4 * kScoreTargetWorkgroups);
  const int per_pass = 64 / score_shape(l.num_kv_heads, l.head_dim).lg;  // blocks per wave pass
  bpw = (bpw + per_pass - 1) / per_pass * per_pass;
  sa.blocks_per_wave = static_cast<int>(bpw > 256 ? 256 : bpw);
  // Summary sets beyond this size are streamed (read once, not worth caching).
  const int64_t summary_bytes = total_blocks * l.num_kv_heads * l.head_dim * 4;
  sa.stream_rows = summary_bytes > kScoreStreamBytes ? 1 : 0;
  sa.top_k = p.top_k;
  sa.keep_num = p.keep_num;
  sa.keep_den = p.keep_den;
  sa.keep_floor = p.keep_floor;
  sa.recent_window = p.recent_window;
  sa.gamma_num = p.gamma_num;
  sa.gamma_den = p.gamma_den;
  TopkArgs ta;
  ta.scores = scores;
  ta.context_lens = context_lens;
  ta.selected = selected;
  ta.num_selected = num_selected;
  ta.spans = spans;
  ta.num_spans = num_spans;
  ta.use_dense = use_dense;
  ta.B = l.batch;
  ta.P = l.block_size;
  ta.max_blocks = l.max_blocks_per_seq;
  ta.top_k = p.top_k;
  ta.keep_num = p.keep_num;
  ta.keep_den = p.keep_den;
  ta.keep_floor = p.keep_floor;
  ta.recent_window = p.recent_window;
  ta.gamma_num = p.gamma_num;
  ta.gamma_den = p.gamma_den;
  if (fused_select_supported(l.max_blocks_per_seq, score_workgroups(sa))) {
    int32_t* counters = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.select_counters);
    return from_hip(launch_score_select(sa, ta, counters, l.dtype, stream));
  }
  hipError_t e = launch_score(sa, l.dtype, stream);
  if (e != hipSuccess) return KVSP_ERR_HIP;
  return from_hip(launch_topk(ta, stream));
}

kvsp_status kvsp_sparse_decode(const kvsp_layout* layout, const kvsp_select_params* params,
                               const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* context_lens,
                               const int32_t* spans, const int32_t* num_spans,
                               const int32_t* selected, const int32_t* num_selected,
                               const int32_t* use_dense, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(layout, params, false, q, k_pool, v_pool, block_table, context_lens, spans,
                    num_spans, selected, num_selected, use_dense, scale, out, lse, workspace,
                    workspace_bytes, stream);
}

kvsp_status kvsp_sparse_decode_noalloc(const kvsp_layout* layout, const kvsp_select_params* params,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       const int32_t* spans, const int32_t* num_spans,
                                       const int32_t* selected, const int32_t* num_selected,
                                       const int32_t* use_dense, float scale, float* out,
                                       float* lse, hipStream_t stream) {
  kvsp_status st = check_decode(layout, params, false, q, k_pool, v_pool, block_table,
                                context_lens, spans, num_spans, selected, num_selected, out);
  if (st != KVSP_OK) return st;
  if (static_decode_bytes(*layout) == 0) return KVSP_ERR_TOO_LARGE;
  DecodeScratch scr;
  if ((st = static_scratch(*layout, stream, &scr)) != KVSP_OK) return st;
  return launch_checked_decode(*layout, params, false, q, k_pool, v_pool, block_table, context_lens,
                               spans, num_spans, selected, num_selected, use_dense, scale, out,
                               lse, scr, stream);
}

kvsp_status kvsp_dense_decode(const kvsp_layout* layout, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* context_lens, float scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(layout, nullptr, true, q, k_pool, v_pool, block_table, context_lens, nullptr,
                    nullptr, nullptr, nullptr, nullptr, scale, out, lse, workspace, workspace_bytes,
                    stream);
}

size_t kvsp_dkv_record_bytes(const kvsp_layout* layout, const kvsp_dkv_params* dkv) {
  if (check_dkv(layout, dkv) != KVSP_OK) return 0;
  return dkv_record_layout(*layout, dkv->n_resid).bytes;
}

size_t kvsp_dkv_workspace_bytes(const kvsp_layout* layout, const kvsp_dkv_params* dkv) {
  if (check_dkv(layout, dkv) != KVSP_OK) return 0;
  return dkv_workspace(*layout).total;
}

kvsp_status kvsp_dkv_compress(const kvsp_layout* layout, const kvsp_dkv_params* dkv,
                              int32_t recent_window, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* context_lens,
                              void* records, hipStream_t stream) {
  kvsp_status st = check_dkv(layout, dkv);
  if (st != KVSP_OK) return st;
  if (recent_window < 0) return KVSP_ERR_INVALID_ARG;
  if (!k_pool || !v_pool || !block_table || !context_lens || !records) return KVSP_ERR_INVALID_ARG;
  const kvsp_layout& l = *layout;
  const DkvRecordLayout r = dkv_record_layout(l, dkv->n_resid);
  DkvCompressArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.records = static_cast<char*>(records);
  a.rec_bytes = static_cast<int64_t>(r.bytes);
  a.off_basis = r.off_basis;
  a.off_coef = r.off_coef;
  a.off_rk = r.off_rk;
  a.off_rv = r.off_rv;
  a.off_ridx = r.off_ridx;
  a.off_rounds = r.off_rounds;
  a.B = l.batch;
  a.Hkv = l.num_kv_heads;
  a.P = l.block_size;
  a.max_blocks = l.max_blocks_per_seq;
  a.num_phys = l.num_phys_blocks;
  a.recent_window = recent_window;
  a.n_resid = dkv->n_resid;
  a.power_iters = dkv->power_iters;  // 0: rounds chosen per block from its Ritz values
  const hipError_t e = launch_dkv_compress(a, l.dtype, l.head_dim, stream);
  if (e == hipErrorNotSupported) return KVSP_ERR_UNSUPPORTED;
  return from_hip(e);
}

kvsp_status kvsp_dkv_decode(const kvsp_layout* layout, const kvsp_select_params* params,
                            const kvsp_dkv_params* dkv, const void* q, const void* k_pool,
                            const void* v_pool, const void* records, const int32_t* block_table,
                            const int32_t* context_lens, const int32_t* selected,
                            const int32_t* num_selected, float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kvsp_status st = check_dkv(layout, dkv);
  if (st != KVSP_OK) return st;
  if (params == nullptr || params->recent_window < 0) return KVSP_ERR_INVALID_ARG;
  if (!q || !k_pool || !v_pool || !records || !block_table || !context_lens || !selected ||
      !num_selected || !out)
    return KVSP_ERR_INVALID_ARG;
  const kvsp_layout& l = *layout;
  const DkvWorkspace ws = dkv_workspace(l);
  if (workspace == nullptr || workspace_bytes < ws.total) return KVSP_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);
  const DkvRecordLayout r = dkv_record_layout(l, dkv->n_resid);
  DkvDecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.records = static_cast<const char*>(records);
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.selected = selected;
  a.num_selected = num_selected;
  a.out = out;
  a.lse = lse;
  a.part_acc = reinterpret_cast<float*>(wsb + ws.part_acc);
  a.part_ml = reinterpret_cast<float*>(wsb + ws.part_ml);
  a.counters = reinterpret_cast<int32_t*>(wsb + ws.counters);
  a.rec_bytes = static_cast<int64_t>(r.bytes);
  a.off_basis = r.off_basis;
  a.off_coef = r.off_coef;
  a.off_rk = r.off_rk;
  a.off_rv = r.off_rv;
  a.off_ridx = r.off_ridx;
  a.B = l.batch;
  a.Hq = l.num_q_heads;
  a.Hkv = l.num_kv_heads;
  a.P = l.block_size;
  a.max_blocks = l.max_blocks_per_seq;
  a.recent_window = params->recent_window;
  a.n_resid = dkv->n_resid;
  a.n_chunks = dkv_chunks(l);
  a.n_wchunks = dkv_window_chunks(l, params->recent_window);
  const float s = scale > 0.f ? scale : 1.0f / __builtin_sqrtf(static_cast<float>(l.head_dim));
  a.scale_log2 = s * 1.4426950408889634f;
  return from_hip(launch_dkv_decode(a, l.dtype, l.head_dim, stream));
}

}  // extern "C"
