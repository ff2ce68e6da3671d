// Compile-time unpack plans for the decode kernel.
//
// A run of 32 consecutive b-bit codes occupies exactly b 32-bit words of the
// LSB-first stream.  For fp16 activations the kernel multiplies codes by
// activations with v_dot2_f32_f16, which takes two 16-bit values per operand.
// A code q with its bits at offset o (o + b <= 10) inside one 16-bit half of a
// 32-bit window is turned into the fp16 value 2^(10-o) + q, exactly, by OR-ing
// the fp16 exponent field (25 - o) above it: the half then reads
// 2^(10-o) * (1 + q*2^o/1024).  One AND-OR therefore converts two codes (one
// per half) at once; one packed subtract of the two constants leaves the
// codes exactly, and one dot2 accumulates x_lo*q_lo + x_hi*q_hi.  (Where both
// codes of a pair sit at one offset -- widths dividing 16 -- the decode kernel
// may instead leave the exponent field zero and read the halves as subnormals.)
//
// Windows: word d shifted right by t*span bits (a funnel shift across words d
// and d+1).  A code whose start lies rel bits into word d (rel < 32) goes to
// the low half (rel < 16) or high half (rel >= 16) of window t = (rel % 16) /
// span at offset (rel % 16) - t*span.  span is chosen so that every offset
// leaves room for the code below bit 10: for b dividing 16 the windows follow
// the code grid (span = b * (floor((10-b)/b) + 1)); otherwise span = 11 - b.
// Inside one window the i-th low code is paired with the i-th high code; a
// half without a code is a dummy (zero mask, activation 0).
#pragma once

namespace lowbit {

struct PairSlot {
  int word;    // source word of the window
  int shift;   // right shift of the window (bits), 0 = the word itself
  int klo;     // code index (0..31) in the low half, -1 = none
  int khi;     // code index in the high half, -1 = none
  int olo;     // bit offset of the low code inside the low half
  int ohi;     // bit offset of the high code inside the high half
};

struct PairTable {
  PairSlot s[32];
  int n;
};

template <int BITS>
struct F16Plan {
  static constexpr int span = (16 % BITS == 0) ? BITS * ((10 - BITS) / BITS + 1) : 11 - BITS;
  static constexpr int wpd = (16 + span - 1) / span;

  static constexpr PairTable build() {
    PairTable tab{};
    tab.n = 0;
    for (int d = 0; d < BITS; ++d) {
      for (int t = 0; t < wpd; ++t) {
        int lo[32] = {}, olo[32] = {}, hi[32] = {}, ohi[32] = {};
        int nlo = 0, nhi = 0;
        for (int k = 0; k < 32; ++k) {
          const int p = k * BITS;
          if (p < 32 * d || p >= 32 * d + 32) continue;
          const int rel = p - 32 * d;
          const int half = rel >= 16 ? 1 : 0;
          const int r16 = rel - 16 * half;
          if (r16 / span != t) continue;
          const int o = r16 - t * span;
          if (half) { hi[nhi] = k; ohi[nhi] = o; ++nhi; }
          else { lo[nlo] = k; olo[nlo] = o; ++nlo; }
        }
        const int np = nlo > nhi ? nlo : nhi;
        for (int i = 0; i < np; ++i) {
          PairSlot& s = tab.s[tab.n++];
          s.word = d;
          s.shift = t * span;
          s.klo = i < nlo ? lo[i] : -1;
          s.olo = i < nlo ? olo[i] : 0;
          s.khi = i < nhi ? hi[i] : -1;
          s.ohi = i < nhi ? ohi[i] : 0;
        }
      }
    }
    return tab;
  }
  static constexpr PairTable table = build();
  static constexpr int n = table.n;
};

// fp16 exponent field that makes bit `o` of the mantissa worth 1.0.
constexpr unsigned f16_magic_for_offset(int o) { return static_cast<unsigned>(25 - o) << 10; }

}  // namespace lowbit
