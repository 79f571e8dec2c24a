// Steps 4 and 5: split-KV attention over the kept blocks plus the exact
// recency window, and the flash-style log-sum-exp merge of the partials (DKV
// abstract). The same kernel is the dense fallback (SparPR news page, "On-
// demand local recomputation with cost-aware fallback") and the dense decode
// ("KV cache offloading", "Why the cache leaves the GPU": a dense step reads
// every stored key and value).
//
// Work decomposition. For sequence b the attended tokens form one ordered
// sequence: the tokens of selected[b][0..k) followed by the window [C*P, L)
// (or all of [0, L) when dense). Given as spans, the same blocks are the
// union of the spans in ascending order (the window run last). Attended
// token i lives in attended block i / P at offset i % P, because every
// attended block but the last is full.
// That sequence is cut into at most max_chunks chunks of whole sub-tiles.
// One workgroup handles one (sequence, KV head, head group, chunk) item: its
// four wavefronts take the chunk's sub-tiles (SUB tokens: 4 KiB of keys and
// as much of values, at least 16 tokens) in turn, each with its own online softmax, and merge
// through LDS at the end. One-head items keep two sub-tiles in flight per
// wavefront, GQA items one; K/V are read non-temporally unless several head
// groups share a KV head.
// Workgroups walk the items with a grid stride, so any mix of sparse and
// dense sequences fills the chip.
//
// Per sub-tile and wavefront:
//   K: 16-byte loads laid out as the A operand of v_mfma_f32_16x16x32_{bf16,
//      f16} (16x16x4 f32 for fp32 caches): row = token, contraction = head
//      dim. The B operand holds the group's queries (up to 16 heads), so the
//      logits of all heads that share a KV head come from one read of K.
//      A pool in host memory (HOSTK) is read row-major instead: each load
//      instruction takes 1 KiB of consecutive rows, which crosses PCIe in
//      larger requests than 64 bytes from each of 16 rows; the wave puts the
//      rows in the A layout through its LDS before the MFMAs.
//   softmax: base-2 online softmax per head; probabilities staged in LDS.
//   V: 16-byte row-major loads (LPR lanes per row); each lane accumulates
//      acc[head][its EPV channels] += p * v in float32.
// A chunk's result is written as a partial (m, l, acc). The last workgroup to
// finish a (sequence, KV head, head group) — counted with one atomic per
// group in the workspace, which that workgroup resets to zero — merges the
// partials by log-sum-exp and writes the output. A sequence that fits in one
// chunk writes its output directly.
// HBM-bound: 2 * D * E bytes per attended token per KV head.

#pragma once

#include "kvsp_device.h"
#include "kvsp_internal.h"

namespace kvsp {

// Bytes of keys a wavefront loads per sub-tile (the same again for values).
#ifndef KVSP_SUB_TILE_BYTES
#define KVSP_SUB_TILE_BYTES 4096
#endif
// Work items of at most this many heads load sub-tile i+1 while they compute
// sub-tile i. Measured: it helps one-head items (little compute per byte,
// registers to spare) and costs GQA items occupancy.
#ifndef KVSP_PIPELINE_MAX_GP
#define KVSP_PIPELINE_MAX_GP 1
#endif
// Groups of at most this many chunks are merged by wave 0 alone, in registers.
constexpr int kFastMergeChunks = 8;
// Chunks per output whose accumulators the merging workgroup requests before
// it has the merge weights.
#ifndef KVSP_MERGE_PRE
#define KVSP_MERGE_PRE 16
#endif
// 1: items are numbered chunk-major (see the item loop of attend_kernel).
#ifndef KVSP_CHUNK_MAJOR
#define KVSP_CHUNK_MAJOR 1
#endif

template <typename T, int D>
struct DecodeShape {
  static constexpr int E = T::kBytes;
  static constexpr int EPV = T::kPerVec;      // elements per 16-byte vector
  static constexpr int LPR = D * E / 16;      // lanes per K/V row
  static constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  static constexpr int NRG = RPL;             // row groups in a wave
  static constexpr int SUB = KVSP_SUB_TILE_BYTES / (D * E) < 16 ? 16 : KVSP_SUB_TILE_BYTES / (D * E);
  static constexpr int TILES = SUB / 16;      // 16-token MFMA tiles per sub-tile
  static constexpr int KLD = D * E / 64;      // K loads per lane per tile
  static constexpr int VLD = SUB / RPL;       // V loads per lane per sub-tile
  static constexpr int PROW = 16;             // floats per token row of p in LDS
};

constexpr int kDecodeWaves = 4;
constexpr int kXcds = 8;  // accelerator complex dies of the MI355X, each with its own L2

struct SeqWork {
  int32_t L, Cw, k, dense, A, T, CT, nc;
};

// A span list's first 64 spans stay in registers from the prologue to the
// first block-id window: per lane (span `lane`), its first logical block, the
// attended blocks before it and its length (0 past the list). `carry` is the
// attended-block count they cover. (Holding more rounds measured as register
// pressure that cost GQA items their second wave per SIMD.) Later spans are
// requested kSpanBatch rounds of 64 at a time.
constexpr int kSpanBatch = 4;
struct SpanRegs {
  int32_t st, ex, ln;
  int32_t n, carry;
};

// (start, end) of span s of sequence b; s must lie in [0, max_blocks].
__device__ __forceinline__ int2 load_span(const DecodeArgs& a, int b, int s) {
  const int64_t i = (static_cast<int64_t>(b) * (a.max_blocks + 1) + s) * 2;
  return *reinterpret_cast<const int2*>(a.spans + i);
}

// Chunking of sequence b's attended tokens: chunks are whole multiples of
// `quantum` tokens (one sub-tile per wavefront), at most max_chunks of them.
// Every lane of the wave calls it (span lists are scanned across the wave).
template <bool SPANS>
__device__ __forceinline__ SeqWork seq_work(const DecodeArgs& a, int b, int quantum,
                                            SpanRegs& sr) {
  SeqWork w;
  const int lane = threadIdx.x % kWave;
  // The plan's loads do not depend on each other and are issued together
  // (one round trip). None sits behind a branch, where it would be waited
  // for alone: an absent array is replaced by context_lens for the load and
  // its value masked afterwards. A span list's first rounds are requested in
  // the same trip (clamped to the row; entries past the count are masked).
  const bool has_flag = a.use_dense != nullptr;
  constexpr bool by_spans = SPANS;
  const int32_t* count = by_spans ? a.num_spans : a.num_selected;
  const bool has_count = count != nullptr;
  w.L = a.context_lens[b];
  const int flag_v = (has_flag ? a.use_dense : a.context_lens)[b];
  const int count_v = (has_count ? count : a.context_lens)[b];
  int2 sp0 = make_int2(0, 0);
  if constexpr (SPANS) sp0 = load_span(a, b, min(lane, a.max_blocks));
  const int flag = has_flag ? flag_v : 0;
  const int cnt = has_count ? count_v : 0;
  const int n = (w.L + a.P - 1) / a.P;
  w.Cw = window_start_block(w.L, a.P, a.recent_window);
  w.dense = a.all_dense || flag != 0;
  if (w.dense) {
    w.k = 0;
    w.A = n;
    w.T = w.L;
  } else if constexpr (SPANS) {
    // A = total length of the spans; inclusive scans give each span the
    // attended blocks before it.
    sr.n = min(cnt, a.max_blocks + 1);
    sr.ln = lane < sr.n ? sp0.y - sp0.x : 0;
    const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(sr.ln)));
    sr.st = sp0.x;
    sr.ex = incl - sr.ln;
    int carry = __builtin_amdgcn_readlane(incl, kWave - 1);
    sr.carry = carry;
    for (int s0 = kWave; s0 < sr.n; s0 += kWave * kSpanBatch) {  // lists past 64 spans
      int2 v[kSpanBatch];
#pragma unroll
      for (int i = 0; i < kSpanBatch; ++i) v[i] = load_span(a, b, min(s0 + kWave * i + lane, a.max_blocks));
#pragma unroll
      for (int i = 0; i < kSpanBatch; ++i) {
        const int len = s0 + kWave * i + lane < sr.n ? v[i].y - v[i].x : 0;
        carry += __builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan(static_cast<uint32_t>(len))),
                                           kWave - 1);
      }
    }
    w.k = 0;
    w.A = carry;
    // every attended block is full except block n - 1, which the window
    // always holds when it is partial
    w.T = w.A > 0 ? w.A * a.P - (n * a.P - w.L) : 0;
  } else {
    w.k = cnt;
    w.A = w.k + (n - w.Cw);
    w.T = w.k * a.P + (w.L - w.Cw * a.P);
  }
  if (w.T > 0) {
    const int per = (w.T + quantum * a.max_chunks - 1) / (quantum * a.max_chunks);
    w.CT = per * quantum;
    w.nc = (w.T + w.CT - 1) / w.CT;
  } else {
    w.CT = quantum;
    w.nc = 1;
  }
  return w;
}

// Physical block of attended block `ab` from the selected list or, when
// dense, the context itself (caller guarantees ab < A).
__device__ __forceinline__ int32_t attended_phys(const DecodeArgs& a, int b, const SeqWork& w,
                                                 int ab) {
  int32_t logical;
  if (w.dense) {
    logical = ab;
  } else if (ab < w.k) {
    logical = a.selected[static_cast<int64_t>(b) * a.max_blocks + ab];
  } else {
    logical = w.Cw + (ab - w.k);
  }
  return a.block_table[static_cast<int64_t>(b) * a.max_blocks + logical];
}

// Span lists: the logical block of attended block gbase + lane. Every span
// that overlaps [gbase, gbase + 64) writes, into the wave's `marks` row at its
// first position in that range, the offset between its logical and attended
// indices; each lane then takes the nearest mark at or below its position.
constexpr int32_t kNoMark = -2147483647 - 1;

__device__ __forceinline__ void span_mark(int32_t* marks, int gbase, int st, int ex, int len) {
  if (len > 0 && ex < gbase + kWave && ex + len > gbase) marks[max(ex - gbase, 0)] = st - ex;
}

// Marks the spans from number s0 on (the attended blocks before s0 are
// `carry`), BATCH rounds of 64 at a time, until the range is covered, then
// resolves every lane. Spans past the range mark nothing.
template <int BATCH>
__device__ __forceinline__ int span_logical_from(const DecodeArgs& a, int b, int n_spans, int s0,
                                                 int carry, int gbase, int32_t* marks) {
  const int lane = threadIdx.x % kWave;
  for (; s0 < n_spans && carry < gbase + kWave; s0 += kWave * BATCH) {
    int2 v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) v[i] = load_span(a, b, min(s0 + kWave * i + lane, a.max_blocks));
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int len = s0 + kWave * i + lane < n_spans ? v[i].y - v[i].x : 0;
      const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(len)));
      span_mark(marks, gbase, v[i].x, carry + incl - len, len);
      carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
  }
  wave_lds_sync();
  const uint64_t below = __ballot(marks[lane] != kNoMark) & (~0ull >> (kWave - 1 - lane));
  const int src = kWave - 1 - __builtin_clzll(below | 1ull);  // lane 0 is marked while gbase < A
  return gbase + lane + marks[src];
}

// First window of an item: span `lane` from registers, later ones in batches.
__device__ __forceinline__ int span_logical_first(const DecodeArgs& a, int b, const SpanRegs& sr,
                                                  int gbase, int32_t* marks) {
  const int lane = threadIdx.x % kWave;
  marks[lane] = kNoMark;
  wave_lds_sync();
  span_mark(marks, gbase, sr.st, sr.ex, sr.ln);
  return span_logical_from<kSpanBatch>(a, b, sr.n, kWave, sr.carry, gbase, marks);
}

// A later window (rare: an item longer than 64 blocks): from the list again,
// one round at a time (this runs inside the streaming loop, where registers
// are scarce).
__device__ __forceinline__ int span_logical_again(const DecodeArgs& a, int b, int n_spans,
                                                  int gbase, int32_t* marks) {
  const int lane = threadIdx.x % kWave;
  wave_lds_sync();  // the previous window's marks have been read
  marks[lane] = kNoMark;
  wave_lds_sync();
  return span_logical_from<1>(a, b, n_spans, 0, 0, gbase, marks);
}

// STREAM: read K/V with non-temporal loads. The launch picks it when every KV
// head is read by one head group only (nothing to reuse from the caches);
// when split head groups share a KV head, default loads let them reuse it.
// SPANS: the kept blocks come as span lists (a.spans), else as selected lists.
// HOSTK: the K pool is host memory (row-major K loads, see above).
template <typename T, int D, int GP, bool STREAM, bool SPANS, bool HOSTK>
__global__ __launch_bounds__(256) void attend_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D>;
  constexpr int E = S::E;
  constexpr int QUANTUM = kDecodeWaves * S::SUB;
  __shared__ float p_lds[kDecodeWaves][S::SUB * S::PROW];
  // One-head items keep the physical ids of 64 consecutive attended blocks in
  // LDS, a row per wave, rather than in a register read with readlane: a
  // refresh load behind a branch makes every later readlane wait at the join
  // for all loads in flight (the prefetched tile included); an LDS read waits
  // for none. (Head-group items measured faster with the register.)
  __shared__ int32_t phys_lds[kDecodeWaves][GP == 1 ? kWave : 1];
  __shared__ int32_t mark_lds[kDecodeWaves][SPANS ? kWave : 1];  // per-wave window marks
  __shared__ float alpha_lds[kDecodeWaves][16];
  __shared__ float ml_lds[kDecodeWaves][2][16];
  __shared__ float xacc[kDecodeWaves][GP * D];
  // HOSTK: a sub-tile's K rows, each padded by 16 bytes so that the reads in
  // the A layout (16 rows at one column) fall in different banks.
  constexpr int KROW = D * E + 16;
  __shared__ __align__(16) char kt_lds[kDecodeWaves][HOSTK ? S::SUB * KROW : 16];
  __shared__ int last_flag;

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hl = lane % 16;  // head within the group (MFMA column)
  const int rg = lane / S::LPR;
  const int col = (lane % S::LPR) * S::EPV;
  const int G = a.Hq / a.Hkv;
  const float NEG_INF = -__builtin_huge_valf();
  const __amdgpu_buffer_rsrc_t part_rsrc =
      coherent_rsrc(a.part_acc, static_cast<uint32_t>(static_cast<int64_t>(a.total_items) * GP * D * sizeof(float)));

  const int n_groups = a.total_items / a.max_chunks;
  for (int wg = blockIdx.x; wg < a.total_items; wg += gridDim.x) {
    // The dispatcher deals consecutive workgroups round-robin to the 8 XCDs
    // (XCD = wg % 8 while the grid is a multiple of 8), each with its own L2.
    // When several head groups read one KV head (xcd_share), the workgroups
    // that share a (sequence, KV head, chunk) get consecutive slots of one
    // XCD, so its L2 serves their common tiles after the first read;
    // otherwise the item is the workgroup index itself.
    int item = wg;
    if (a.xcd_share) {
      const int slot = wg / kXcds;
      const int hg_w = slot % a.n_head_groups;
      const int unit = (slot / a.n_head_groups) * kXcds + wg % kXcds;  // (pair, chunk), chunk-major
      const int n_pairs = n_groups / a.n_head_groups;
      const int c_w = unit / n_pairs;
      const int pair = unit - c_w * n_pairs;
      item = c_w * n_groups + pair * a.n_head_groups + hg_w;
    }
#if KVSP_CHUNK_MAJOR
    // Chunk-major order: consecutive workgroups (which the dispatcher deals
    // round-robin to the XCDs) take the same chunk of different groups, so
    // every XCD gets an equal share of first and last chunks.
    const int c = item / n_groups;
    int rest = item - c * n_groups;
#else
    int rest = item;
    const int c = rest % a.max_chunks;
    rest /= a.max_chunks;
#endif
    const int grp = rest;  // (b * Hkv + g) * n_head_groups + hg
    const int hg = rest % a.n_head_groups;
    rest /= a.n_head_groups;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;
    // Queries of this head group as the MFMA B operand, loaded before the
    // sequence's plan so both travel in the same round trip.
    const int head_in_group = hg * GP + hl;
    const bool head_ok = hl < GP && head_in_group < G;
    const int hq_lane = g * G + head_in_group;
    uint4 qop[S::KLD];
#pragma unroll
    for (int s = 0; s < S::KLD; ++s) {
      if (head_ok) {
        const char* qp = static_cast<const char*>(a.q) +
                         (static_cast<int64_t>(b * a.Hq + hq_lane) * D + k_elem_offset<T>(lane, s)) * E;
        qop[s] = load16(qp);
      } else {
        qop[s] = make_uint4(0, 0, 0, 0);
      }
    }
    SpanRegs sr;
    const SeqWork w = seq_work<SPANS>(a, b, QUANTUM, sr);
    const bool by_spans = SPANS && !w.dense;  // uniform
    if (c >= w.nc) continue;  // uniform over the workgroup
    const int start = c * w.CT;
    const int end = min(w.T, start + w.CT);

    float m_run = NEG_INF, l_run = 0.f;
    float acc[GP][S::EPV];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < S::EPV; ++e) acc[h][e] = 0.f;

    // Physical ids of 64 consecutive attended blocks, one per lane.
    const int first_tok = start + wave * S::SUB;
    int gbase = min(first_tok, max(end - 1, 0)) / a.P;
    int phys_v = 0;
    {
      const int ab = gbase + lane;
      int32_t p0;
      if (SPANS && by_spans) {
        const int logical = span_logical_first(a, b, sr, gbase, mark_lds[wave]);
        p0 = ab < w.A ? a.block_table[static_cast<int64_t>(b) * a.max_blocks + logical] : 0;
      } else {
        p0 = ab < w.A ? attended_phys(a, b, w, ab) : 0;
      }
      if constexpr (GP == 1) {
        phys_lds[wave][lane] = p0;
        wave_lds_sync();
      } else {
        phys_v = p0;
      }
    }

    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);

    struct SubTile {
      uint4 kv[S::TILES][S::KLD];
      uint4 vv[S::VLD];
    };

    // Per-lane byte offsets inside a 16-row tile (loop invariant): K in the MFMA
    // A-operand layout (row hl, 16 bytes per lane group, 64 bytes per step),
    // V row-major (row group rg, channels col..col+EPV).
    // HOSTK: load s of a 16-row tile is its bytes [1024 s, 1024 s + 1024),
    // lane i taking 16 of them.
    const uint32_t k_lane_off =
        HOSTK ? static_cast<uint32_t>(16 * lane) : static_cast<uint32_t>(hl * D * E + (lane / 16) * 16);
    constexpr int K_STEP = HOSTK ? 1024 : 64;
    const uint32_t v_lane_off = static_cast<uint32_t>((rg * D + col) * E);

    auto kv_load = [](const char* p) {
      if constexpr (STREAM) {
        return load16_stream(p);
      } else {
        return load16(p);
      }
    };
    // Enqueue the K and V loads of the sub-tile starting at attended token i0.
    // Tile bases are wave-uniform, so every load is base + lane offset.
    // A repeat (repeat == true, the one-head pipeline past the end) keeps
    // the instruction count, which the waits depend on, but points every
    // lane at the tile's first 16 bytes: one line per load instead of the
    // tile, whose data would not be used.
    auto issue = [&](int i0, SubTile& st, bool repeat = false) {
      const uint32_t k_off = repeat ? 0u : k_lane_off;
      const uint32_t v_off = repeat ? 0u : v_lane_off;
      const int a_last = (min(i0 + S::SUB, end) - 1) / a.P;
      if (a_last - gbase >= kWave) {
        gbase = i0 / a.P;
        const int ab = gbase + lane;
        int32_t p1;
        if (SPANS && by_spans) {
          const int logical = span_logical_again(a, b, sr.n, gbase, mark_lds[wave]);
          p1 = ab < w.A ? a.block_table[static_cast<int64_t>(b) * a.max_blocks + logical] : 0;
        } else {
          p1 = ab < w.A ? attended_phys(a, b, w, ab) : 0;
        }
        if constexpr (GP == 1) {
          phys_lds[wave][lane] = p1;
          wave_lds_sync();
        } else {
          phys_v = p1;
        }
      }
      int64_t tile_byte0[S::TILES];  // byte offset of the tile's first row in the pool
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        const int ti = i0 + 16 * t;
        const int ab = min(ti, end - 1) / a.P;
        int64_t phys;
        if constexpr (GP == 1) {
          phys = phys_lds[wave][ab - gbase];
        } else {
          phys = __builtin_amdgcn_readlane(phys_v, ab - gbase);
        }
        tile_byte0[t] = ((phys * a.Hkv + g) * a.P + (ti % a.P)) * static_cast<int64_t>(D * E);
      }
      // Rows past `end` still lie inside a valid physical block (tiles are
      // 16-row aligned, P >= 16): they are loaded unconditionally, their
      // logits are masked to -inf and their values zeroed before use.
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        const char* tk = kbase + tile_byte0[t];
#pragma unroll
        for (int s = 0; s < S::KLD; ++s) st.kv[t][s] = kv_load(tk + k_off + (repeat ? 0 : K_STEP * s));
      }
#pragma unroll
      for (int r = 0; r < S::VLD; ++r) {
        const int t = (r * S::RPL) / 16;
        const char* tv = vbase + tile_byte0[t] + (r * S::RPL - 16 * t) * D * E;
        st.vv[r] = kv_load(tv + v_off);
      }
    };

    // Online-softmax update with the sub-tile starting at attended token i0.
    auto consume = [&](int i0, const SubTile& st) {
      // HOSTK: the row-major K goes through the wave's LDS into the A layout,
      // the same 16 bytes per lane and step that the direct loads hold.
      uint4 kt[S::TILES][S::KLD];
      if constexpr (HOSTK) {
        char* kb = kt_lds[wave];
#pragma unroll
        for (int t = 0; t < S::TILES; ++t)
#pragma unroll
          for (int s = 0; s < S::KLD; ++s) {
            const int byte = 1024 * s + 16 * lane;  // within the tile's 16 * D * E bytes
            const int row = 16 * t + byte / (D * E);
            *reinterpret_cast<uint4*>(kb + row * KROW + byte % (D * E)) = st.kv[t][s];
          }
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < S::TILES; ++t)
#pragma unroll
          for (int s = 0; s < S::KLD; ++s)
            kt[t][s] = *reinterpret_cast<const uint4*>(kb + (16 * t + hl) * KROW + 64 * s + 16 * (lane / 16));
        wave_lds_sync();  // read before the next sub-tile is written
      } else {
#pragma unroll
        for (int t = 0; t < S::TILES; ++t)
#pragma unroll
          for (int s = 0; s < S::KLD; ++s) kt[t][s] = st.kv[t][s];
      }
      // Logits (base 2): lane holds head hl, tokens 16*t + 4*(lane/16) + i.
      float s2[S::TILES][4];
      float mloc = NEG_INF;
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
        floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S::KLD; ++s) sc = QkMfma<T>::step(kt[t][s], qop[s], sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) s2[t][i] = sc[i] * a.scale_log2;
      }
      // Tokens past `end` exist only in a chunk's last sub-tile (wave-uniform).
      if (i0 + S::SUB > end) {
#pragma unroll
        for (int t = 0; t < S::TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i0 + 16 * t + 4 * (lane / 16) + i >= end) s2[t][i] = NEG_INF;
      }
#pragma unroll
      for (int t = 0; t < S::TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s2[t][i]);
      mloc = fold_max<16>(mloc);  // over the four lanes holding head hl
      const float m_new = fmaxf(m_run, mloc);
      const bool none = m_new == NEG_INF;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < S::TILES; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = none ? 0.f : __builtin_amdgcn_exp2f(s2[t][i] - m_new);
          psum += pv;
          p_lds[wave][(16 * t + 4 * (lane / 16) + i) * S::PROW + hl] = pv;
        }
      }
      psum = fold_sum<16>(psum);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (lane < 16) alpha_lds[wave][hl] = alpha;
      wave_lds_sync();

      // alpha is exactly 1 for every head whose running max did not move, and
      // scaling by 1 changes no bit: the rescale is skipped when that holds
      // for all heads (wave-uniform).
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float al = alpha_lds[wave][h];
#pragma unroll
          for (int e = 0; e < S::EPV; ++e) acc[h][e] *= al;
        }
      }
      // Rows past `end` (only in a chunk's last sub-tile, wave-uniform) may
      // hold any bits: their packed values are zeroed before use.
      uint4 vraw[S::VLD];
#pragma unroll
      for (int r = 0; r < S::VLD; ++r) vraw[r] = st.vv[r];
      if (i0 + S::SUB > end) {
#pragma unroll
        for (int r = 0; r < S::VLD; ++r)
          if (i0 + r * S::RPL + rg >= end) vraw[r] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < S::VLD; ++r) {
        const int rr = r * S::RPL + rg;
        float vf[S::EPV];
        T::widen(vraw[r], vf);
        const float* prow = &p_lds[wave][rr * S::PROW];
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float ph = prow[h];
#pragma unroll
          for (int e = 0; e < S::EPV; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        }
      }
      wave_lds_sync();
    };

    constexpr int STRIDE = kDecodeWaves * S::SUB;  // the four waves take turns
    SubTile buf0, buf1;
    int i0 = first_tok;
    if (i0 < end) issue(i0, buf0);
    if constexpr (GP <= KVSP_PIPELINE_MAX_GP) {
      if constexpr (GP == 1) {
        // One-head items: every step issues a tile, so that every path has
        // the same loads in flight and a tile's use waits for that tile alone
        // (with a conditional issue the wait also covers the first load of
        // the tile just requested). Past the end the current tile is
        // requested again (valid addresses; the data is not used).
        while (i0 < end) {
          const int i1 = i0 + STRIDE;
          issue(i1 < end ? i1 : i0, buf1, i1 >= end);
          consume(i0, buf0);
          if (i1 >= end) break;
          const int i2 = i1 + STRIDE;
          issue(i2 < end ? i2 : i1, buf0, i2 >= end);
          consume(i1, buf1);
          i0 = i2;
        }
      } else {
        while (i0 < end) {
          const int i1 = i0 + STRIDE;
          if (i1 < end) issue(i1, buf1);
          consume(i0, buf0);
          if (i1 >= end) break;
          const int i2 = i1 + STRIDE;
          if (i2 < end) issue(i2, buf0);
          consume(i1, buf1);
          i0 = i2;
        }
      }
    } else {
      while (i0 < end) {
        consume(i0, buf0);
        i0 += STRIDE;
        if (i0 < end) issue(i0, buf0);
      }
    }

    // Fold the row groups: every lane then holds its wave's sums for its channels.
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < S::EPV; ++e) acc[h][e] = fold_sum<S::LPR>(acc[h][e]);

    // Merge the four wavefronts. Each leaves its (m, l) per head and its
    // unscaled sums for the heads its row groups own in LDS; after one
    // barrier every thread takes OPT consecutive outputs (one head, channels
    // d0 .. d0 + OPT) and combines the four waves: M = max_w m_w, weights
    // 2^(m_w - M), summed in wave order. The outputs (or the chunk's partial)
    // are thus written by all four waves at once.
    if (lane < 16) {
      ml_lds[wave][0][hl] = m_run;
      ml_lds[wave][1][hl] = l_run;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h % S::NRG != rg) continue;
#pragma unroll
      for (int e = 0; e < S::EPV; ++e) xacc[wave][h * D + col + e] = acc[h][e];
    }
    __syncthreads();
    {
      constexpr int OUTS = GP * D;
      constexpr int OPT = OUTS >= 2048 ? 8 : (OUTS >= 256 ? OUTS / 256 : 1);
      const int o0 = threadIdx.x * OPT;
      if (o0 < OUTS) {
        const int h = o0 / D;
        const int d0 = o0 % D;
        float mw[kDecodeWaves], lw[kDecodeWaves];
        float M = NEG_INF;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) {
          mw[v] = ml_lds[v][0][h];
          lw[v] = ml_lds[v][1][h];
          M = fmaxf(M, mw[v]);
        }
        float o[OPT];
#pragma unroll
        for (int e = 0; e < OPT; ++e) o[e] = 0.f;
        float Ls = 0.f;
#pragma unroll
        for (int v = 0; v < kDecodeWaves; ++v) {
          const float wv = M == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mw[v] - M);
          Ls += lw[v] * wv;
#pragma unroll
          for (int e = 0; e < OPT; ++e) o[e] += xacc[v][o0 + e] * wv;
        }
        const int hq = g * G + hg * GP + h;
        if (hg * GP + h < G) {
          if (w.nc == 1) {
            const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
            float* dst = a.out + (static_cast<int64_t>(b) * a.Hq + hq) * D + d0;
#pragma unroll
            for (int e = 0; e < OPT; ++e) dst[e] = o[e] * inv;
            if (d0 == 0 && a.lse != nullptr)
              a.lse[static_cast<int64_t>(b) * a.Hq + hq] =
                  Ls > 0.f ? (M + __builtin_log2f(Ls)) * 0.69314718055994531f : NEG_INF;
          } else {
            const int64_t slot = static_cast<int64_t>(grp) * a.max_chunks + c;
            const uint32_t off = static_cast<uint32_t>(((slot * GP + h) * D + d0) * sizeof(float));
            if constexpr (OPT >= 4) {
#pragma unroll
              for (int e = 0; e < OPT; e += 4)
                store_coherent4(part_rsrc, off + e * sizeof(float), make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]));
            } else {
#pragma unroll
              for (int e = 0; e < OPT; ++e) store_coherent1(part_rsrc, off + e * sizeof(float), o[e]);
            }
          }
        }
        if (w.nc > 1 && d0 == 0) {
          const int64_t slot = static_cast<int64_t>(grp) * a.max_chunks + c;
          store_coherent(a.part_ml + (slot * GP + h) * 2 + 0, M);
          store_coherent(a.part_ml + (slot * GP + h) * 2 + 1, Ls);
        }
      }
      if (w.nc > 1) wait_stores_done();  // the partial is at the device coherence point before it is counted
    }
    if (w.nc > 1) {
      __syncthreads();
      if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(a.counters + grp, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == w.nc - 1;
      }
      __syncthreads();
      if (last_flag) {
        if (GP <= S::NRG && w.nc <= kFastMergeChunks) {
          // Few chunks and at most one head per row group: each output lane
          // of wave 0 (row group = head, EPV channels) loads every chunk's
          // (m, l) and its channels in one round trip and merges them in
          // registers; no LDS, no barrier.
          const int h = rg;
          if (wave == 0 && h < GP && hg * GP + h < G) {
            const int64_t slot0 = static_cast<int64_t>(grp) * a.max_chunks;
            float4 pa[kFastMergeChunks][S::EPV / 4];
            float pm[kFastMergeChunks], pl[kFastMergeChunks];
#pragma unroll
            for (int cc = 0; cc < kFastMergeChunks; ++cc) {
              pm[cc] = NEG_INF;
              pl[cc] = 0.f;
#pragma unroll
              for (int q = 0; q < S::EPV / 4; ++q) pa[cc][q] = make_float4(0.f, 0.f, 0.f, 0.f);
              if (cc < w.nc) {
                const int64_t ps = (slot0 + cc) * GP + h;
#pragma unroll
                for (int q = 0; q < S::EPV / 4; ++q)
                  pa[cc][q] = load_coherent4(part_rsrc, static_cast<uint32_t>((ps * D + col + 4 * q) * sizeof(float)));
                pm[cc] = load_coherent(a.part_ml + ps * 2);
                pl[cc] = load_coherent(a.part_ml + ps * 2 + 1);
              }
            }
            float M = NEG_INF;
#pragma unroll
            for (int cc = 0; cc < kFastMergeChunks; ++cc)
              if (pl[cc] > 0.f) M = fmaxf(M, pm[cc]);
            float Ls = 0.f;
            float o[S::EPV];
#pragma unroll
            for (int e = 0; e < S::EPV; ++e) o[e] = 0.f;
            if (M != NEG_INF) {
#pragma unroll
              for (int cc = 0; cc < kFastMergeChunks; ++cc) {
                if (pl[cc] > 0.f) {
                  const float wgt = __builtin_amdgcn_exp2f(pm[cc] - M);
                  Ls += pl[cc] * wgt;
#pragma unroll
                  for (int q = 0; q < S::EPV / 4; ++q) {
                    o[4 * q + 0] += wgt * pa[cc][q].x;
                    o[4 * q + 1] += wgt * pa[cc][q].y;
                    o[4 * q + 2] += wgt * pa[cc][q].z;
                    o[4 * q + 3] += wgt * pa[cc][q].w;
                  }
                }
              }
            }
            const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
            const int hq = g * G + hg * GP + h;
            float* dst = a.out + (static_cast<int64_t>(b) * a.Hq + hq) * D + col;
#pragma unroll
            for (int q = 0; q < S::EPV / 4; ++q)
              *reinterpret_cast<float4*>(dst + 4 * q) =
                  make_float4(o[4 * q] * inv, o[4 * q + 1] * inv, o[4 * q + 2] * inv, o[4 * q + 3] * inv);
            if (col == 0 && a.lse != nullptr)
              a.lse[static_cast<int64_t>(b) * a.Hq + hq] =
                  Ls > 0.f ? (M + __builtin_log2f(Ls)) * 0.69314718055994531f : NEG_INF;
          }
        } else {
          // Every chunk of this group is published: merge by log-sum-exp,
          // reading the partials at the device coherence point.
          //   1. the first MERGE_PRE chunks' accumulators of every output this
          //      thread owns are requested at once (16-byte loads);
          //   2. meanwhile each wave takes heads h = wave, wave + 4, ...: lane
          //      cc reads (m, l) of chunk cc, and wave reductions give
          //      M = max m, the weights 2^(m - M) (0 for empty chunks, kept in
          //      LDS) and Lsum = sum l 2^(m - M);
          //   3. out = sum weight * acc / Lsum, the chunks split over CG thread
          //      groups, folded through LDS.
          // The merge reuses the LDS of the main loop (xacc and p_lds).
          const int64_t slot0 = static_cast<int64_t>(grp) * a.max_chunks;
          float* wt_s = &xacc[0][0];                   // [max_chunks][GP] weights
          float* head_s = wt_s + a.max_chunks * GP;    // [GP][2]: M, Lsum
          float4* red_s = reinterpret_cast<float4*>(&p_lds[0][0]);
          constexpr int PAIRS = GP * D / 4;                     // (head, 4 channels) outputs
          constexpr int CG = PAIRS >= 256 ? 1 : 256 / PAIRS;    // chunk groups per output
          constexpr int PER = PAIRS >= 256 ? PAIRS / 256 : 1;   // outputs per thread
          constexpr int PRE = KVSP_MERGE_PRE;
          const int cg = threadIdx.x / (PAIRS >= 256 ? 256 : PAIRS);
          const int pbase = threadIdx.x % (PAIRS >= 256 ? 256 : PAIRS);
          auto acc_off = [&](int cc, int pv) {
            const int h = (4 * pv) / D;
            const int d = (4 * pv) % D;
            return static_cast<uint32_t>((((slot0 + cc) * GP + h) * D + d) * sizeof(float));
          };
          float4 pre[PER][PRE];
  #pragma unroll
          for (int q = 0; q < PER; ++q)
  #pragma unroll
            for (int i = 0; i < PRE; ++i) {
              const int cc = cg + i * CG;
              pre[q][i] = cc < w.nc ? load_coherent4(part_rsrc, acc_off(cc, pbase + q * 256))
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            }
          constexpr int HPW = (GP + kDecodeWaves - 1) / kDecodeWaves;  // heads per wave
          float mv[HPW], lv[HPW];
  #pragma unroll
          for (int i = 0; i < HPW; ++i) {
            const int h = wave + i * kDecodeWaves;
            mv[i] = NEG_INF;
            lv[i] = 0.f;
            if (h < GP && lane < w.nc) {
              mv[i] = load_coherent(a.part_ml + ((slot0 + lane) * GP + h) * 2);
              lv[i] = load_coherent(a.part_ml + ((slot0 + lane) * GP + h) * 2 + 1);
            }
          }
  #pragma unroll
          for (int i = 0; i < HPW; ++i) {
            const int h = wave + i * kDecodeWaves;
            if (h < GP) {  // wave-uniform
              const float M = group_max<kWave>(lv[i] > 0.f ? mv[i] : NEG_INF);
              const float wt = (lv[i] > 0.f && M != NEG_INF) ? __builtin_amdgcn_exp2f(mv[i] - M) : 0.f;
              const float Ls = group_sum<kWave>(lv[i] * wt);
              if (lane < w.nc) wt_s[lane * GP + h] = wt;
              if (lane == 0) {
                head_s[2 * h] = M;
                head_s[2 * h + 1] = Ls;
              }
            }
          }
          __syncthreads();
  #pragma unroll
          for (int q = 0; q < PER; ++q) {
            const int pv = pbase + q * 256;
            const int h = (4 * pv) / D;
            const int d = (4 * pv) % D;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  #pragma unroll
            for (int i = 0; i < PRE; ++i) {
              const int cc = cg + i * CG;
              if (cc < w.nc) {
                const float wgt = wt_s[cc * GP + h];
                o.x += wgt * pre[q][i].x;
                o.y += wgt * pre[q][i].y;
                o.z += wgt * pre[q][i].z;
                o.w += wgt * pre[q][i].w;
              }
            }
  #pragma unroll 8
            for (int cc = cg + PRE * CG; cc < w.nc; cc += CG) {
              const float wgt = wt_s[cc * GP + h];
              const float4 pa = load_coherent4(part_rsrc, acc_off(cc, pv));
              o.x += wgt * pa.x;
              o.y += wgt * pa.y;
              o.z += wgt * pa.z;
              o.w += wgt * pa.w;
            }
            if constexpr (CG > 1) {
              red_s[threadIdx.x] = o;
            }
            __syncthreads();
            if (cg == 0 && hg * GP + h < G) {
              if constexpr (CG > 1) {
                for (int k = 1; k < CG; ++k) {
                  const float4 r = red_s[k * PAIRS + pbase];
                  o.x += r.x;
                  o.y += r.y;
                  o.z += r.z;
                  o.w += r.w;
                }
              }
              const float M = head_s[2 * h];
              const float Ls = head_s[2 * h + 1];
              const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
              const int hq = g * G + hg * GP + h;
              *reinterpret_cast<float4*>(a.out + (static_cast<int64_t>(b) * a.Hq + hq) * D + d) =
                  make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
              if (d == 0 && a.lse != nullptr)
                a.lse[static_cast<int64_t>(b) * a.Hq + hq] =
                    Ls > 0.f ? (M + __builtin_log2f(Ls)) * 0.69314718055994531f : NEG_INF;
            }
            __syncthreads();
          }
        }
        if (threadIdx.x == 0) store_coherent_i(a.counters + grp, 0);  // ready for the next call
      }
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

template <typename T, int D, int GP, bool SPANS, bool HOSTK>
static hipError_t launch_decode_s(const DecodeArgs& a, int num_wgs, hipStream_t stream) {
  if (a.n_head_groups == 1) {
    hipLaunchKernelGGL((attend_kernel<T, D, GP, true, SPANS, HOSTK>), dim3(num_wgs),
                       dim3(kDecodeWaves * kWave), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attend_kernel<T, D, GP, false, SPANS, HOSTK>), dim3(num_wgs),
                       dim3(kDecodeWaves * kWave), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D, int GP, bool HOSTK>
static hipError_t launch_decode_t(const DecodeArgs& a, int num_wgs, hipStream_t stream) {
  return a.spans != nullptr ? launch_decode_s<T, D, GP, true, HOSTK>(a, num_wgs, stream)
                            : launch_decode_s<T, D, GP, false, HOSTK>(a, num_wgs, stream);
}

template <typename T, int D, bool HOSTK>
static hipError_t launch_decode_d(const DecodeArgs& a, int gp, int num_wgs, hipStream_t stream) {
  switch (gp) {
    case 1: return launch_decode_t<T, D, 1, HOSTK>(a, num_wgs, stream);
    case 2: return launch_decode_t<T, D, 2, HOSTK>(a, num_wgs, stream);
    case 4: return launch_decode_t<T, D, 4, HOSTK>(a, num_wgs, stream);
    case 8: return launch_decode_t<T, D, 8, HOSTK>(a, num_wgs, stream);
    default: return launch_decode_t<T, D, 16, HOSTK>(a, num_wgs, stream);
  }
}

template <typename T, bool HOSTK>
static hipError_t launch_decode_dt(const DecodeArgs& a, int gp, int num_wgs, hipStream_t stream) {
  return a.D == 64 ? launch_decode_d<T, 64, HOSTK>(a, gp, num_wgs, stream)
                   : launch_decode_d<T, 128, HOSTK>(a, gp, num_wgs, stream);
}

// Every instantiation of attend_kernel for one kind of K pool (HOSTK: host
// memory); each kind is compiled in a translation unit of its own.
template <bool HOSTK>
static hipError_t launch_decode_kind(const DecodeArgs& a, int dtype, int group_pad, int num_wgs,
                                     hipStream_t stream) {
  if (dtype == KVSP_F32) return launch_decode_dt<F32, HOSTK>(a, group_pad, num_wgs, stream);
  if (dtype == KVSP_F16) return launch_decode_dt<F16, HOSTK>(a, group_pad, num_wgs, stream);
  return launch_decode_dt<BF16, HOSTK>(a, group_pad, num_wgs, stream);
}

}  // namespace kvsp
