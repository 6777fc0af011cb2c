// N-gram hash oracle: a plain CPU implementation of the Engram hash step.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
// call this file. It shares no code with the GPU library.
//
// Source of the method: the zhichai.net TileKernels page, section
// "5. Engram — 条件记忆门控": engram_hash combines the token ids of an N-gram
// with XOR and multiplication into a hash value and maps it to an index of
// an embedding table; there are 2 N-gram layers, N up to 3, and 8 tables per
// layer. The page fixes nothing else, so the rest is a reading, stated here
// (the plainest one: the caller's constants, the usual modulus map):
//
//   * token ids are int32, taken as their 32-bit unsigned pattern;
//   * layer l uses the last n_l tokens of the sequence up to and including
//     position s; positions before the start of the sequence read `pad`;
//   * table j of layer l has odd 64-bit multipliers a[l][j][i] (drawn by the
//     caller) and a size M[l][j]; the hash is
//         h = XOR over i < n_l of ( tok(s - i) * a[l][j][i]  mod 2^64 )
//     and the index is  h mod M[l][j];
//   * the result is int32 [B, S, L, K], row-major.
//
// Everything is exact unsigned integer arithmetic; there is no rounding.

#include <cstdint>

namespace {

uint64_t ngram_hash(const int32_t* seq, int64_t s, int n, const uint64_t* a,
                    uint32_t pad) {
  uint64_t h = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t p = s - i;
    const uint32_t tok = p >= 0 ? (uint32_t)seq[p] : pad;
    h ^= (uint64_t)tok * a[i];  // unsigned wrap-around is mod 2^64
  }
  return h;
}

}  // namespace

extern "C" {

// tokens int32 [B, S]; ngram int32 [L]; mult uint64 [L, K, 4] (entries
// i >= n_l unused); table_size uint32 [L, K]; out int32 [B, S, L, K].
void oracle_engram_hash(const int32_t* tokens, int64_t B, int64_t S, int L,
                        int K, const int32_t* ngram, const uint64_t* mult,
                        const uint32_t* table_size, uint32_t pad,
                        int32_t* out) {
  for (int64_t b = 0; b < B; ++b) {
    const int32_t* seq = tokens + b * S;
    for (int64_t s = 0; s < S; ++s) {
      int32_t* o = out + (b * S + s) * L * K;
      for (int l = 0; l < L; ++l)
        for (int j = 0; j < K; ++j) {
          const uint64_t h = ngram_hash(seq, s, ngram[l], mult + (l * K + j) * 4, pad);
          o[l * K + j] = (int32_t)(h % (uint64_t)table_size[l * K + j]);
        }
    }
  }
}

}  // extern "C"
