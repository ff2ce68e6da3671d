// Host harness for the decode kernel's fp16 slot plans (qmv_plan.h).
//
// Reads, from stdin, a bit width b and runs of b 32-bit words (the packed
// LSB-first code stream of 32 codes each, as decimal numbers) and prints, for
// every run and every slot of the width's plan, the 32-bit word the kernel
// multiplies: "run slot klo khi offset word".  The word is formed from the
// plan tables the way the kernel forms it: a funnel shift of two stream words
// (v_alignbit_b32), or a byte gather from two source words (v_perm_b32: bytes
// 0-3 of S1, then 4-7 of S0), then the mask of the two codes.  A test compares
// the two halves with the oracle's unpacked codes.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "qmv_plan.h"

using namespace lowbit;

// Bits [q, q + 32) of the run's stream (zero past its end).
static uint32_t stream_word(const uint32_t* w, int bits, int q) {
  const int d = q / 32, sh = q % 32;
  if (d >= bits) return 0u;
  const uint64_t lo = w[d];
  const uint64_t hi = d + 1 < bits ? w[d + 1] : 0u;
  return static_cast<uint32_t>(((hi << 32) | lo) >> sh);
}

static uint32_t byte_perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  const uint64_t v = (static_cast<uint64_t>(s0) << 32) | s1;
  uint32_t out = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (sel >> (8 * i)) & 0xffu;
    if (b > 7) return 0xffffffffu;   // (the plans only select bytes 0-7)
    out |= static_cast<uint32_t>((v >> (8 * b)) & 0xffu) << (8 * i);
  }
  return out;
}

template <int BITS>
static void emit(const std::vector<uint32_t>& words) {
  using S = F16Slots<BITS>;
  constexpr uint32_t m = (1u << BITS) - 1u;
  const size_t runs = words.size() / BITS;
  for (size_t r = 0; r < runs; ++r) {
    const uint32_t* w = &words[r * BITS];
    for (int i = 0; i < S::n; ++i) {
      uint32_t word;
      const int o = S::offset(i);
      if constexpr (16 % BITS == 0) {
        const PairSlot s = S::Plan::table.s[i];
        const uint32_t mask = (s.klo >= 0 ? (m << s.olo) : 0u) | (s.khi >= 0 ? (m << (16 + s.ohi)) : 0u);
        word = stream_word(w, BITS, 32 * s.word + s.shift) & mask;
      } else {
        const PermSlot s = S::Plan::table.s[i];
        const uint32_t mask = (m << s.o) | (m << (16 + s.o));
        word = byte_perm(stream_word(w, BITS, s.q0), stream_word(w, BITS, s.q1), s.sel) & mask;
      }
      std::printf("%zu %d %d %d %d %u\n", r, i, S::klo(i), S::khi(i), o, word);
    }
  }
}

int main() {
  int bits = 0;
  if (std::scanf("%d", &bits) != 1) return 2;
  std::vector<uint32_t> words;
  unsigned v;
  while (std::scanf("%u", &v) == 1) words.push_back(v);
  if (bits < 1 || bits > 7 || words.size() % bits != 0) return 2;
  switch (bits) {
    case 1: emit<1>(words); break;
    case 2: emit<2>(words); break;
    case 3: emit<3>(words); break;
    case 4: emit<4>(words); break;
    case 5: emit<5>(words); break;
    case 6: emit<6>(words); break;
    case 7: emit<7>(words); break;
  }
  return 0;
}
