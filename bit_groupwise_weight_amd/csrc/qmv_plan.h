// Compile-time unpack plans for the decode kernel (fp16 activations).
//
// A run of 32 consecutive b-bit codes occupies exactly b 32-bit words of the
// LSB-first stream.  The kernel multiplies codes by activations with
// v_dot2_f32_f16, which takes two 16-bit values per operand, so each slot of a
// plan is one 32-bit word holding two codes, one per 16-bit half, and the
// staged activation word of the same slot holds their two activations.
//
// Codes enter the dot products as fp16 subnormals: a half whose only set bits
// are a code q at bit offset o, with o + b <= 11, reads as q * 2^(o-24)
// exactly (below bit 10 the half is a subnormal; with bit 10 set it is the
// first normal binade, whose step is still 2^-24).  v_dot2_f32_f16 keeps
// subnormal inputs, and x * q * 2^(o-24) is exact in fp32, so the products of
// one offset share an fp32 accumulator and the accumulators are combined by
// exact power-of-two scalings, sum x*q = sum_o acc_o * 2^(24-o).  A slot only
// needs its two codes at the same offset of their halves.
//
// Two plans place them there:
//   * F16Plan (widths dividing 16: 1, 2, 4): window t of word d is the word
//     shifted right by t*span bits (a funnel shift across words d and d+1);
//     its low and high halves are 16 bits apart, a whole number of codes, so
//     the i-th low code and the i-th high code share an offset.  span is a
//     multiple of b (at most 10): fewer, wider windows mean fewer shifts but
//     more distinct offsets to combine.
//   * F16PermPlan (3, 5, 6, 7 bits): 16 bits is no whole number of codes, so
//     the two halves are gathered separately, with one byte permute
//     (v_perm_b32) from two source words.  Code k is paired with k + D, where
//     D*b is a multiple of 8 (D = 8 / gcd(b, 8)): both codes lie at the same
//     bit position within a byte, and their halves start the same number of
//     bits before them.  A half starts at the byte boundary at or below its
//     code, or 4 bits above that boundary when the code would otherwise reach
//     past bit 10 (its source words are then the stream shifted by 4 bits,
//     one funnel shift each).  Where the two halves do not fit in two
//     consecutive source words, each half comes from a word of its own.
// Every slot is then masked down to its two codes and multiplied with one
// dot2.
#pragma once

#include <stdint.h>

namespace lowbit {

// ------------------------------------------------- funnel-shift windows --

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
constexpr int f16_default_span() {
  return BITS * ((10 - BITS) / BITS + 1);
}

// Windows of SPAN bits, codes on the grid of the window.
template <int BITS, int SPAN = f16_default_span<BITS>()>
struct F16Plan {
  static_assert(16 % BITS == 0, "the two halves of a window must be whole codes apart");
  static_assert(SPAN % BITS == 0 && SPAN >= BITS && SPAN <= 10,
                "every offset leaves room for the code below bit 10");
  static constexpr int span = SPAN;
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

// ------------------------------------------------------- byte permutes --

struct PermSlot {
  int klo, khi;   // codes in the low and the high half
  int o;          // their common bit offset inside the halves
  int q1, q0;     // stream bit at which source words S1 and S0 start
  uint32_t sel;   // v_perm_b32 selector: bytes 0-3 of S1, then 4-7 of S0
};

struct PermTable {
  PermSlot s[16];
  int n;
};

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

template <int BITS>
struct F16PermPlan {
  static_assert(16 % BITS != 0 && BITS < 8, "widths dividing 16 take the funnel-shift plan");
  static constexpr int D = 8 / gcd_int(BITS, 8);   // partner distance in codes

  static constexpr PermTable build() {
    PermTable tab{};
    tab.n = 0;
    for (int k = 0; k < 32; ++k) {
      if ((k / D) % 2 != 0) continue;               // the partner of k - D
      const int p = BITS * k;
      int o = p % 8;
      if (o + BITS > 11) o -= 4;
      const int plo = p - o, phi = plo + BITS * D;  // start bits of the halves
      const int base = plo % 8;                     // 0, or 4: shifted source words
      const int ul = plo - base, uh = phi - base;   // byte-aligned in that stream
      const int dl = ul / 32;
      PermSlot& s = tab.s[tab.n++];
      s.klo = k;
      s.khi = k + D;
      s.o = o;
      int bl = 0, bh = 0;
      if (uh + 16 <= 32 * dl + 64) {                // both halves in words dl, dl + 1
        s.q1 = 32 * dl + base;
        s.q0 = 32 * (dl + 1) + base;
        bl = (ul - 32 * dl) / 8;
        bh = (uh - 32 * dl) / 8;
      } else {
        if (ul % 32 <= 16) { s.q1 = 32 * dl + base; bl = (ul % 32) / 8; }
        else { s.q1 = plo; bl = 0; }
        if (uh % 32 <= 16) { s.q0 = 32 * (uh / 32) + base; bh = 4 + (uh % 32) / 8; }
        else { s.q0 = phi; bh = 4; }
      }
      s.sel = static_cast<uint32_t>(bl) | (static_cast<uint32_t>(bl + 1) << 8) |
              (static_cast<uint32_t>(bh) << 16) | (static_cast<uint32_t>(bh + 1) << 24);
    }
    return tab;
  }
  static constexpr PermTable table = build();
  static constexpr int n = table.n;
};

// ---------------------------------------------------- plan of a width --

// The fp16 slot plan of a width: funnel-shift windows for the widths dividing
// 16 (at 1 bit, windows of 4 bits: four offsets to combine instead of ten; at
// 2 bits, of 8: four offsets instead of five, same shifts), byte permutes for
// the others.  klo/khi: the codes of slot i; offset: their
// common bit offset.
template <int BITS, bool PERM = (16 % BITS != 0)> struct F16Slots;
template <int BITS> struct F16Slots<BITS, false> {
  static constexpr int span = BITS == 1 ? 4 : BITS == 2 ? 8 : f16_default_span<BITS>();
  using Plan = F16Plan<BITS, span>;
  static constexpr int n = Plan::n;
  static constexpr int klo(int i) { return Plan::table.s[i].klo; }
  static constexpr int khi(int i) { return Plan::table.s[i].khi; }
  static constexpr int offset(int i) {
    return Plan::table.s[i].klo >= 0 ? Plan::table.s[i].olo : Plan::table.s[i].ohi;
  }
};
template <int BITS> struct F16Slots<BITS, true> {
  using Plan = F16PermPlan<BITS>;
  static constexpr int n = Plan::n;
  static constexpr int klo(int i) { return Plan::table.s[i].klo; }
  static constexpr int khi(int i) { return Plan::table.s[i].khi; }
  static constexpr int offset(int i) { return Plan::table.s[i].o; }
};

}  // namespace lowbit
