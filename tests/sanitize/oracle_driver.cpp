// Host-only driver for running the C++ oracle under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_oracle_sanitized.py with
// g++). It calls every exported oracle routine on small seeded inputs of each
// storage type, including the edge cases: an empty sequence, a context inside
// the recent window, the dense fallback, k >= C, exact ties, a shuffled block
// table, appends that complete a block, and the threaded decode step.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
int kvsp_oracle_abi_version();
void kvsp_oracle_widen(int dtype, const void* src, int64_t n, double* dst);
void kvsp_oracle_plan(int32_t L, int32_t P, int32_t W, int32_t top_k, int32_t keep_num,
                      int32_t keep_den, int32_t keep_floor, int32_t gamma_num, int32_t gamma_den,
                      int32_t* out);
void kvsp_oracle_summaries(int dtype, const void* k_pool, int32_t B, int32_t Hkv, int32_t P,
                           int32_t D, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* ctx_lens, double* summ);
void kvsp_oracle_append(int dtype, void* k_pool, void* v_pool, int32_t Hkv, int32_t P, int32_t D,
                        const void* k_new, const void* v_new, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* positions, int32_t B, double* filled,
                        int32_t* flags);
void kvsp_oracle_decode_step(int dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                             int32_t max_blocks, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* ctx_lens, const double* summ, int32_t top_k,
                             int32_t keep_num, int32_t keep_den, int32_t keep_floor,
                             int32_t recent_window, int32_t gamma_num, int32_t gamma_den,
                             double scale, const uint8_t* head_mask, int32_t* plan,
                             double* scores, int32_t* sel, int32_t* spans, int32_t* nspans,
                             double* out, double* lse, int32_t threads);
}

namespace {

uint64_t state = 0x243F6A8885A308D3ull;
uint32_t next_u32() {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return static_cast<uint32_t>(state >> 33);
}

// Finite values of each storage type (0 fp32, 1 fp16, 2 bf16); `flat` makes
// every element equal so that scores tie exactly.
std::vector<uint8_t> values(int dtype, size_t n, bool flat) {
  const size_t e = dtype == 0 ? 4 : 2;
  std::vector<uint8_t> out(n * e);
  for (size_t i = 0; i < n; ++i) {
    const uint32_t r = flat ? 0x9E3779B9u : next_u32();
    if (dtype == 0) {
      const float f = static_cast<float>(static_cast<int32_t>(r % 2001) - 1000) / 500.0f;
      std::memcpy(&out[i * 4], &f, 4);
    } else {
      // sign, an exponent below the all-ones pattern, any mantissa
      const uint16_t exp_max = dtype == 1 ? 30 : 254;
      const uint16_t exp_lo = dtype == 1 ? 10 : 120;
      const uint16_t mant_bits = dtype == 1 ? 10 : 7;
      const uint16_t ex = static_cast<uint16_t>(exp_lo + (r >> 8) % (exp_max - exp_lo + 1 > 8 ? 8 : 1));
      const uint16_t bits = static_cast<uint16_t>(((r & 1u) << 15) | (ex << mant_bits) |
                                                  ((r >> 16) & ((1u << mant_bits) - 1)));
      std::memcpy(&out[i * 2], &bits, 2);
    }
  }
  return out;
}

int run_case(int dtype, bool flat, int threads) {
  const int32_t B = 4, Hq = 4, Hkv = 2, D = 32, P = 16, max_blocks = 8, phys = B * max_blocks;
  const int32_t ctx[B] = {0, 11, 77, 128};  // empty, inside the window, ragged, full table
  std::vector<int32_t> table(B * max_blocks);
  for (int32_t i = 0; i < B * max_blocks; ++i) table[i] = i;
  for (int32_t i = B * max_blocks - 1; i > 0; --i) {  // shuffled pool
    const int32_t j = static_cast<int32_t>(next_u32() % (i + 1));
    std::swap(table[i], table[j]);
  }
  auto kp = values(dtype, static_cast<size_t>(phys) * Hkv * P * D, flat);
  auto vp = values(dtype, static_cast<size_t>(phys) * Hkv * P * D, false);
  auto q = values(dtype, static_cast<size_t>(B) * Hq * D, flat);
  std::vector<double> wide(static_cast<size_t>(B) * Hq * D);
  kvsp_oracle_widen(dtype, q.data(), static_cast<int64_t>(wide.size()), wide.data());
  std::vector<double> summ(static_cast<size_t>(B) * max_blocks * Hkv * D, 0.0);
  kvsp_oracle_summaries(dtype, kp.data(), B, Hkv, P, D, table.data(), max_blocks, ctx, summ.data());

  struct Sel { int32_t top_k, keep_num, keep_den, floor, W, gnum, gden; };
  const Sel sels[] = {
      {3, 1, 1, 1, 20, 1, 1},    // top-k with a window
      {0, 1, 2, 2, 0, 1, 1},     // keep ratio, no window
      {0, 7, 10, 1, 16, 3, 5},   // dense fallback
      {99, 1, 1, 1, 8, 1, 1},    // k >= C
      {0, 0, 1, 0, 40, 1, 1},    // window only
  };
  for (const Sel& s : sels) {
    std::vector<int32_t> plan(B * 5), sel(B * max_blocks, -1), spans(B * (max_blocks + 1) * 2, -1),
        nspans(B);
    std::vector<double> scores(B * max_blocks, 0.0), out(static_cast<size_t>(B) * Hq * D),
        lse(B);
    lse.resize(B * Hq);
    std::vector<uint8_t> mask(B * Hq, 1);
    mask[1] = 0;
    kvsp_oracle_decode_step(dtype, B, Hq, Hkv, D, P, max_blocks, q.data(), kp.data(), vp.data(),
                            table.data(), ctx, summ.data(), s.top_k, s.keep_num, s.keep_den,
                            s.floor, s.W, s.gnum, s.gden, 0.0, mask.data(), plan.data(),
                            scores.data(), sel.data(), spans.data(), nspans.data(), out.data(),
                            lse.data(), threads);
  }
  int32_t plan_out[5];
  kvsp_oracle_plan(0, P, 0, 0, 1, 1, 0, 1, 1, plan_out);
  kvsp_oracle_plan(1 << 30, 1 << 10, 7, 0, 1, 3, 5, 1, 2, plan_out);

  // append one token per sequence, the last one completing its block
  const int32_t pos[B] = {-1, 11, 77, 127};
  auto kn = values(dtype, static_cast<size_t>(B) * Hkv * D, false);
  auto vn = values(dtype, static_cast<size_t>(B) * Hkv * D, false);
  std::vector<double> filled(static_cast<size_t>(B) * Hkv * D);
  std::vector<int32_t> flags(B);
  kvsp_oracle_append(dtype, kp.data(), vp.data(), Hkv, P, D, kn.data(), vn.data(), table.data(),
                     max_blocks, pos, B, filled.data(), flags.data());
  return flags[3] == 1 ? 0 : 1;
}

}  // namespace

int main() {
  if (kvsp_oracle_abi_version() != 1) return 1;
  int bad = 0;
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int flat = 0; flat < 2; ++flat)
      for (int threads : {1, 3}) bad |= run_case(dtype, flat != 0, threads);
  std::printf(bad ? "driver: unexpected result\n" : "driver ok\n");
  return bad;
}
