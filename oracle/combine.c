/*
 * Plain C part of the CPU oracle: the consumer's top-k weighted combine,
 * accumulated exactly as the definition states, in binary32 with one fused
 * multiply-add per pick, picks in ascending k.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the oracle package (itself used only by
 * the tests, the package smoke check and the benchmark's CPU baseline).  The
 * HIP library neither links nor calls it, and it shares no code with it.
 *
 * Follows "P3PeerSendConfig" (Mojo struct page), description: the combine
 * kernel reads the slot of pick src_topk of token src_idx from the rank's
 * receive buffer and weights it by the token's routing weight; and
 * "ep_signal_completion" (Mojo function page), description: the consumer
 * reads a rank's slots once the rank is complete.
 *
 * For token i the caller lists its local picks p in [first[i], first[i+1]),
 * in ascending pick order, each with its routing weight weight[p] (binary32)
 * and its slot row slots[p][0..n) (bf16 codes).  The result is
 *     acc = +0;  for each pick p in order:  acc = fmaf(weight[p], slot[p][j], acc)
 * per column j, written to out[i][j] as binary32 (rounded to bf16 by the
 * caller).  A token with no local pick gets +0.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16_value(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16; /* bf16 = upper half of a binary32 */
  float v;
  memcpy(&v, &bits, sizeof v);
  return v;
}

void oracle_combine_fmaf(const uint16_t* slots, const float* weight, const int64_t* first,
                         int64_t n_tokens, int64_t n, float* out) {
  for (int64_t i = 0; i < n_tokens; ++i) {
    float* acc = out + i * n;
    for (int64_t j = 0; j < n; ++j) acc[j] = 0.0f;
    for (int64_t p = first[i]; p < first[i + 1]; ++p) {
      const uint16_t* row = slots + p * n;
      const float w = weight[p];
      for (int64_t j = 0; j < n; ++j) acc[j] = fmaf(w, bf16_value(row[j]), acc[j]);
    }
  }
}
