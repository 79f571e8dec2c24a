// Reference oracle for query-aware sparse block decode attention.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, plain, double-precision
// statement of what the GPU library computes. It exists so that tests, the
// smoke check and the benchmark's CPU baseline have something independent to
// compare against. No product code path may link, load or call it; it shares
// no source, header, helper or constant with the HIP library.
//
// Sources followed (page titles and sections; the pages define no API):
//   [SparPR-QA]   "SparPR: Runtime KV-Cache Recovery for Resource-Constrained LLM
//                 Inference on Consumer Hardware" (aimodeling.com news page),
//                 section "Three decisions rather than one compression ratio",
//                 paragraph "Query-Aware key-block selection".
//   [SparPR-BUD]  same page and section, paragraph "Dynamic budget control"
//                 (the Minimum Keep Floor).
//   [SparPR-REC]  same page and section, paragraph "On-demand local
//                 recomputation with cost-aware fallback" (spans, threshold γ).
//   [DKV]         "DKV: Anchor + Low-Rank Differential KV-Cache Compression for
//                 Scalable Long-Context Inference", abstract (exact recency
//                 window, flash-style log-sum-exp merge of partial attentions).
//   [KVO-WHY]     "KV cache offloading" (aiwiki), section "Why the cache leaves
//                 the GPU" (dense decode reads every stored key and value).
//   [SparPR-INTRO] the SparPR page's opening paragraphs (the KV cache gains
//                 one token per decoded token).
//
// Arithmetic: every stored element (fp32, fp16 or bf16) is widened exactly to
// double, and everything after that is double. Loops run in the plain order
// the definitions state; there is no blocking, no fusion and no reordering.
//
// Data layout (shared convention with the library's public header, restated
// here on purpose rather than included):
//   q          [B][Hq][D]                    element type `dtype`
//   K, V pool  [num_phys][Hkv][P][D]         element type `dtype`
//   block table[B][max_blocks]  int32        logical block -> physical block
//   context    [B]              int32        tokens cached per sequence
// dtype codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16.
//
// Parity pins for every function live in tests/test_oracle_*.py.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>
#include <algorithm>

namespace {

// ---- element widening --------------------------------------------------------

// IEEE 754 binary16 -> double, from the format definition: 1 sign bit,
// 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal,
// exponent 31 is infinity / NaN.
double half_bits_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 0x1F;
  const int frac = h & 0x3FF;
  double mag;
  if (expo == 0) {
    mag = std::ldexp(static_cast<double>(frac), -24);            // frac * 2^-14 * 2^-10
  } else if (expo == 31) {
    mag = frac == 0 ? std::numeric_limits<double>::infinity()
                    : std::numeric_limits<double>::quiet_NaN();
  } else {
    mag = std::ldexp(static_cast<double>(1024 + frac), expo - 25); // (1 + f/1024) * 2^(e-15)
  }
  return sign ? -mag : mag;
}

// bfloat16 is the upper half of an IEEE binary32.
double bf16_bits_to_double(uint16_t b) {
  const uint32_t w = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return static_cast<double>(f);
}

double load_elem(int dtype, const void* base, int64_t i) {
  if (dtype == 0) {
    float f;
    std::memcpy(&f, static_cast<const char*>(base) + 4 * i, sizeof f);
    return static_cast<double>(f);
  }
  uint16_t b;
  std::memcpy(&b, static_cast<const char*>(base) + 2 * i, sizeof b);
  return dtype == 1 ? half_bits_to_double(b) : bf16_bits_to_double(b);
}

// Element index of K/V(phys, g, t, d) in the [num_phys][Hkv][P][D] pool.
int64_t pool_index(int64_t phys, int64_t g, int64_t t, int64_t d, int64_t Hkv, int64_t P,
                   int64_t D) {
  return ((phys * Hkv + g) * P + t) * D + d;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

int kvsp_oracle_abi_version() { return 1; }

// Widen n stored elements to double (exposed so the tests can pin the
// conversions against independent decoders).
void kvsp_oracle_widen(int dtype, const void* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(dtype, src, i);
}

// ---- step 3, integer part: how many blocks, which are candidates, k ---------
//
// For a sequence of L cached tokens in blocks of P tokens:
//   n   = ceil(L / P) logical blocks.
//   The exact recency window [DKV] is the token range [C*P, L) with
//   C = floor(max(0, L - W) / P): the last W tokens, widened down to a block
//   boundary so that the blocks before it are whole. Those C older blocks
//   are the candidates that [SparPR-QA] scores.
//   k_req = top_k if top_k > 0, else ceil(C * keep_num / keep_den) (a keep
//           ratio given as an exact fraction; integer arithmetic).
//   k_eff = min(max(k_req, keep_floor), C)   — the Minimum Keep Floor bounds
//           the budget from below [SparPR-BUD]; there are only C candidates.
//   use_dense = C > 0 and k_eff / C > gamma_num / gamma_den: above the Dense
//           Fallback Threshold γ the kept fraction is too large for the
//           sparse path to pay off, and the step goes dense [SparPR-REC].
// out = {n, C, k_req, k_eff, use_dense}.
void kvsp_oracle_plan(int32_t L, int32_t P, int32_t W, int32_t top_k, int32_t keep_num,
                      int32_t keep_den, int32_t keep_floor, int32_t gamma_num,
                      int32_t gamma_den, int32_t* out) {
  const int64_t n = ceil_div(L, P);
  const int64_t hist = std::max<int64_t>(0, static_cast<int64_t>(L) - W);
  const int64_t C = hist / P;
  int64_t k_req;
  if (top_k > 0) {
    k_req = top_k;
  } else {
    k_req = ceil_div(C * keep_num, keep_den);
  }
  int64_t k_eff = std::max<int64_t>(k_req, keep_floor);
  k_eff = std::min<int64_t>(k_eff, C);
  const int64_t use_dense =
      (C > 0 && k_eff * static_cast<int64_t>(gamma_den) > static_cast<int64_t>(gamma_num) * C) ? 1
                                                                                              : 0;
  out[0] = static_cast<int32_t>(n);
  out[1] = static_cast<int32_t>(C);
  out[2] = static_cast<int32_t>(k_req);
  out[3] = static_cast<int32_t>(k_eff);
  out[4] = static_cast<int32_t>(use_dense);
}

// ---- step 1: block summary [SparPR-QA] ---------------------------------------
//
// The summary of a block for one KV head is the mean key vector over the
// block's P tokens: s[d] = (1/P) * sum_t K[phys][g][t][d].
void kvsp_oracle_block_summary(int dtype, const void* k_pool, int32_t Hkv, int32_t P,
                               int32_t D, int32_t phys, int32_t g, double* s) {
  for (int32_t d = 0; d < D; ++d) {
    double sum = 0.0;
    for (int32_t t = 0; t < P; ++t) sum += load_elem(dtype, k_pool, pool_index(phys, g, t, d, Hkv, P, D));
    s[d] = sum / static_cast<double>(P);
  }
}

// Summaries for a batch, indexed by LOGICAL block: summ[B][max_blocks][Hkv][D].
// Written for every full block j < floor(L_b / P) of every sequence; other
// entries are left as they are.
void kvsp_oracle_summaries(int dtype, const void* k_pool, int32_t B, int32_t Hkv, int32_t P,
                           int32_t D, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* ctx_lens, double* summ) {
  for (int32_t b = 0; b < B; ++b) {
    const int32_t full = ctx_lens[b] / P;
    for (int32_t j = 0; j < full && j < max_blocks; ++j) {
      const int32_t phys = block_table[static_cast<int64_t>(b) * max_blocks + j];
      for (int32_t g = 0; g < Hkv; ++g) {
        double* s = summ + ((static_cast<int64_t>(b) * max_blocks + j) * Hkv + g) * D;
        kvsp_oracle_block_summary(dtype, k_pool, Hkv, P, D, phys, g, s);
      }
    }
  }
}

// ---- decode-time append [SparPR-INTRO, SparPR-QA] ----------------------------
//
// One decode step adds one token per sequence [SparPR-INTRO]. For sequence b
// with positions[b] = p >= 0, the new key and value rows (k_new/v_new
// [B][Hkv][D], element type `dtype`) are copied into token p % P of physical
// block block_table[b][p / P], for every KV head. If p % P == P - 1 the token
// completes its block, which therefore now has a summary [SparPR-QA]: the
// mean key of its P tokens, computed with kvsp_oracle_block_summary on the
// updated pool, goes to filled[b][g][d] and flags[b] = 1. Otherwise (or when
// p < 0: no token this step) nothing is written for b and flags[b] = 0.
// Pools are modified in place.
void kvsp_oracle_append(int dtype, void* k_pool, void* v_pool, int32_t Hkv, int32_t P,
                        int32_t D, const void* k_new, const void* v_new,
                        const int32_t* block_table, int32_t max_blocks,
                        const int32_t* positions, int32_t B, double* filled, int32_t* flags);

// ---- step 2: block relevance score [SparPR-QA] -------------------------------
//
// score[j] = sum over query heads h (ascending) of <q[h], s[j][g(h)]>, where
// query head h reads KV head g(h) = h / (Hq / Hkv) (grouped-query attention;
// with Hq == Hkv this is one summary per head). No 1/sqrt(D): the ranking is
// what matters. q_b is one sequence's [Hq][D]; summ_b its [max_blocks][Hkv][D].
void kvsp_oracle_scores(int dtype, const void* q_b, const double* summ_b, int32_t Hq,
                        int32_t Hkv, int32_t D, int32_t C, double* score) {
  const int32_t G = Hq / Hkv;
  for (int32_t j = 0; j < C; ++j) {
    double total = 0.0;
    for (int32_t h = 0; h < Hq; ++h) {
      const int32_t g = h / G;
      const double* s = summ_b + (static_cast<int64_t>(j) * Hkv + g) * D;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += load_elem(dtype, q_b, static_cast<int64_t>(h) * D + d) * s[d];
      total += dot;
    }
    score[j] = total;
  }
}

// ---- step 3: Top-k [SparPR-QA] ------------------------------------------------
//
// The k blocks that rank highest by (score descending, block index ascending),
// returned in ascending block order. Equal scores go to the lower index.
void kvsp_oracle_topk(const double* score, int32_t C, int32_t k, int32_t* sel) {
  std::vector<int32_t> order(static_cast<size_t>(C));
  for (int32_t j = 0; j < C; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(),
                   [score](int32_t a, int32_t b) { return score[a] > score[b]; });
  std::vector<int32_t> chosen(order.begin(), order.begin() + k);
  std::sort(chosen.begin(), chosen.end());
  for (int32_t i = 0; i < k; ++i) sel[i] = chosen[i];
}

// ---- step 3: span merge [SparPR-REC] ------------------------------------------
//
// Maximal runs of consecutive logical block ids in (selected blocks) ∪ (window
// blocks [C, n)), as half-open [start, end) pairs in ascending order. The
// window run is last; it joins the last selected run when that run ends at
// C - 1. Returns the number of spans written to spans[2*i], spans[2*i+1].
int32_t kvsp_oracle_spans(const int32_t* sel, int32_t k, int32_t C, int32_t n, int32_t* spans) {
  std::vector<int32_t> ids(sel, sel + k);
  for (int32_t j = C; j < n; ++j) ids.push_back(j);
  int32_t count = 0;
  size_t i = 0;
  while (i < ids.size()) {
    size_t e = i + 1;
    while (e < ids.size() && ids[e] == ids[e - 1] + 1) ++e;
    spans[2 * count] = ids[i];
    spans[2 * count + 1] = ids[e - 1] + 1;
    ++count;
    i = e;
  }
  return count;
}

// ---- step 4: partial softmax over a token subset [DKV] -----------------------
//
// For one query head (vector q_h, KV head g) and a list of logical token
// positions `tokens` of one sequence (block table row bt_row):
//   z_t = scale * <q_h, K(t)>,  m = max_t z_t,  l = sum_t exp(z_t - m),
//   acc[d] = sum_t exp(z_t - m) * V(t)[d],
// with K(t) = Kpool[bt_row[t / P]][g][t % P]. An empty list gives m = -inf,
// l = 0, acc = 0.
void kvsp_oracle_partial(int dtype, const void* q_h, const void* k_pool, const void* v_pool,
                         int32_t Hkv, int32_t P, int32_t D, int32_t g, const int32_t* bt_row,
                         const int32_t* tokens, int32_t ntok, double scale, double* m, double* l,
                         double* acc) {
  std::vector<double> z(static_cast<size_t>(ntok));
  double mx = -std::numeric_limits<double>::infinity();
  for (int32_t i = 0; i < ntok; ++i) {
    const int32_t t = tokens[i];
    const int64_t phys = bt_row[t / P];
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d)
      dot += load_elem(dtype, q_h, d) * load_elem(dtype, k_pool, pool_index(phys, g, t % P, d, Hkv, P, D));
    z[i] = scale * dot;
    mx = std::max(mx, z[i]);
  }
  double sum = 0.0;
  for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
  for (int32_t i = 0; i < ntok; ++i) {
    const int32_t t = tokens[i];
    const int64_t phys = bt_row[t / P];
    const double w = std::exp(z[i] - mx);
    sum += w;
    for (int32_t d = 0; d < D; ++d)
      acc[d] += w * load_elem(dtype, v_pool, pool_index(phys, g, t % P, d, Hkv, P, D));
  }
  *m = mx;
  *l = sum;
}

// ---- step 5: log-sum-exp merge of partials [DKV] ------------------------------
//
// Given partials (m_i, l_i, acc_i) over disjoint token subsets:
//   M = max_i m_i,  Lsum = sum_i l_i * exp(m_i - M),
//   out = sum_i acc_i * exp(m_i - M) / Lsum,  lse = M + ln(Lsum).
// Empty partials (l_i = 0, m_i = -inf) contribute nothing. If every partial is
// empty, out = 0 and lse = -inf.
void kvsp_oracle_merge(int32_t nparts, const double* m, const double* l, const double* acc,
                       int32_t D, double* out, double* lse) {
  double M = -std::numeric_limits<double>::infinity();
  for (int32_t i = 0; i < nparts; ++i)
    if (l[i] > 0.0) M = std::max(M, m[i]);
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (M == -std::numeric_limits<double>::infinity()) {
    *lse = M;
    return;
  }
  double Lsum = 0.0;
  for (int32_t i = 0; i < nparts; ++i) {
    if (!(l[i] > 0.0)) continue;
    const double w = std::exp(m[i] - M);
    Lsum += l[i] * w;
    for (int32_t d = 0; d < D; ++d) out[d] += acc[static_cast<int64_t>(i) * D + d] * w;
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= Lsum;
  *lse = M + std::log(Lsum);
}

// ---- steps 4-5 for one (sequence, query head) over an explicit token list ----
//
// Single pass softmax attention: a partial over the whole list, then a merge
// of that one partial (which is the normalisation).
void kvsp_oracle_attend_tokens(int dtype, const void* q_h, const void* k_pool,
                               const void* v_pool, int32_t Hkv, int32_t P, int32_t D, int32_t g,
                               const int32_t* bt_row, const int32_t* tokens, int32_t ntok,
                               double scale, double* out, double* lse) {
  std::vector<double> acc(static_cast<size_t>(D));
  double m, l;
  kvsp_oracle_partial(dtype, q_h, k_pool, v_pool, Hkv, P, D, g, bt_row, tokens, ntok, scale, &m,
                      &l, acc.data());
  kvsp_oracle_merge(1, &m, &l, acc.data(), D, out, lse);
}

// The attended token positions of one sequence: with use_dense every token
// [0, L) [SparPR-REC, KVO-WHY]; otherwise the tokens of the selected blocks
// followed by the exact window [C*P, L) [DKV]. Returns the count; `tokens`
// must hold L entries.
int32_t kvsp_oracle_attended_tokens(int32_t L, int32_t P, int32_t C, const int32_t* sel,
                                    int32_t k, int32_t use_dense, int32_t* tokens) {
  int32_t count = 0;
  if (use_dense) {
    for (int32_t t = 0; t < L; ++t) tokens[count++] = t;
    return count;
  }
  for (int32_t i = 0; i < k; ++i)
    for (int32_t t = sel[i] * P; t < sel[i] * P + P; ++t) tokens[count++] = t;
  for (int32_t t = C * P; t < L; ++t) tokens[count++] = t;
  return count;
}

// ---- one whole decode step for a batch ---------------------------------------
//
// Steps 2-5 (and the dense fallback) for every sequence, given summaries
// (double, by logical block, from kvsp_oracle_summaries). Select parameters
// as in kvsp_oracle_plan. Outputs (all host arrays):
//   plan      [B][5]            {n, C, k_req, k_eff, use_dense}
//   scores    [B][max_blocks]   score of candidate j < C (rest untouched)
//   sel       [B][max_blocks]   ascending selected ids (first k_eff)
//   spans     [B][max_blocks+1][2], nspans [B]
//   out       [B][Hq][D], lse [B][Hq] — only for (b, h) with head_mask[b*Hq+h]
//             != 0 (head_mask NULL means all).
// scale <= 0 means 1/sqrt(D). The (sequence, query head) attentions are
// independent; `threads` > 1 spreads them over that many host threads
// (OpenMP) without changing what each one computes.
void kvsp_oracle_decode_step(int dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t P, int32_t max_blocks, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* ctx_lens, const double* summ, int32_t top_k,
                             int32_t keep_num, int32_t keep_den, int32_t keep_floor,
                             int32_t recent_window, int32_t gamma_num, int32_t gamma_den,
                             double scale, const uint8_t* head_mask, int32_t* plan,
                             double* scores, int32_t* sel, int32_t* spans, int32_t* nspans,
                             double* out, double* lse, int32_t threads) {
  const int64_t elem = dtype == 0 ? 4 : 2;
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(D));
  const int32_t G = Hq / Hkv;
  std::vector<std::vector<int32_t>> tokens(static_cast<size_t>(B));
  std::vector<int32_t> ntok(static_cast<size_t>(B));
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = ctx_lens[b];
    int32_t* pl = plan + 5 * b;
    kvsp_oracle_plan(L, P, recent_window, top_k, keep_num, keep_den, keep_floor, gamma_num,
                     gamma_den, pl);
    const int32_t n = pl[0], C = pl[1], k = pl[3], dense = pl[4];
    const char* q_b = static_cast<const char*>(q) + static_cast<int64_t>(b) * Hq * D * elem;
    const double* summ_b = summ + static_cast<int64_t>(b) * max_blocks * Hkv * D;
    double* score_b = scores + static_cast<int64_t>(b) * max_blocks;
    int32_t* sel_b = sel + static_cast<int64_t>(b) * max_blocks;
    kvsp_oracle_scores(dtype, q_b, summ_b, Hq, Hkv, D, C, score_b);
    kvsp_oracle_topk(score_b, C, k, sel_b);
    nspans[b] = kvsp_oracle_spans(sel_b, k, C, n,
                                  spans + static_cast<int64_t>(b) * (max_blocks + 1) * 2);
    tokens[b].resize(static_cast<size_t>(L));
    ntok[b] = kvsp_oracle_attended_tokens(L, P, C, sel_b, k, dense, tokens[b].data());
  }
  const int64_t pairs = static_cast<int64_t>(B) * Hq;
#pragma omp parallel for num_threads(threads > 1 ? threads : 1) schedule(dynamic, 1)
  for (int64_t i = 0; i < pairs; ++i) {
    if (head_mask && !head_mask[i]) continue;
    const int32_t b = static_cast<int32_t>(i / Hq), h = static_cast<int32_t>(i % Hq);
    const char* q_h = static_cast<const char*>(q) + i * D * elem;
    kvsp_oracle_attend_tokens(dtype, q_h, k_pool, v_pool, Hkv, P, D, h / G,
                              block_table + static_cast<int64_t>(b) * max_blocks,
                              tokens[b].data(), ntok[b], scale, out + i * D, lse + i);
  }
}

void kvsp_oracle_append(int dtype, void* k_pool, void* v_pool, int32_t Hkv, int32_t P,
                        int32_t D, const void* k_new, const void* v_new,
                        const int32_t* block_table, int32_t max_blocks,
                        const int32_t* positions, int32_t B, double* filled, int32_t* flags) {
  const int64_t elem = dtype == 0 ? 4 : 2;
  for (int32_t b = 0; b < B; ++b) {
    flags[b] = 0;
    const int32_t p = positions[b];
    if (p < 0) continue;
    const int32_t j = p / P;
    const int32_t t = p % P;
    const int32_t phys = block_table[static_cast<int64_t>(b) * max_blocks + j];
    for (int32_t g = 0; g < Hkv; ++g) {
      const int64_t src = (static_cast<int64_t>(b) * Hkv + g) * D;
      const int64_t dst = pool_index(phys, g, t, 0, Hkv, P, D);
      std::memcpy(static_cast<char*>(k_pool) + dst * elem,
                  static_cast<const char*>(k_new) + src * elem, D * elem);
      std::memcpy(static_cast<char*>(v_pool) + dst * elem,
                  static_cast<const char*>(v_new) + src * elem, D * elem);
    }
    if (t == P - 1) {
      flags[b] = 1;
      for (int32_t g = 0; g < Hkv; ++g)
        kvsp_oracle_block_summary(dtype, k_pool, Hkv, P, D, phys, g,
                                  filled + (static_cast<int64_t>(b) * Hkv + g) * D);
    }
  }
}

}  // extern "C"
