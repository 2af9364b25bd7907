// Host check of the expansion table of the 16:32 product on the dense matrix instruction
// (nm_skinny_impl.h). For every mask byte (which columns of 8 a lane's fragment keeps) and
// every start offset of the lane's 8-half window, the 4 output dwords built from the table
// entry must hold the byte's kept values in ascending column order at their columns and
// zeros at the other columns. The byte selection of v_perm_b32 is emulated from its
// definition (selector bytes 0..3 pick bytes of the second source, 4..7 of the first, 12 a
// zero byte).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "nm_skinny_impl.h"

using nm::skinny_detail::ExpandTable;

static uint32_t perm(uint32_t a, uint32_t b, uint32_t sel, bool* ok) {
  const uint64_t d = (uint64_t(a) << 32) | b;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const unsigned s = (sel >> (8 * i)) & 0xFF;
    uint32_t byte = 0;
    if (s < 8) byte = uint32_t(d >> (8 * s)) & 0xFF;
    else if (s != 12) *ok = false;
    r |= byte << (8 * i);
  }
  return r;
}

int main() {
  static const ExpandTable t = nm::skinny_detail::make_expand_table();
  int failures = 0, cases = 0;
  // a packed word of 16 distinct nonzero halves, and the window of 8 starting at `pc`
  uint16_t word[24];
  for (int i = 0; i < 24; ++i) word[i] = uint16_t(0x3C00 + 37 * i + 3);
  for (int b = 0; b < 256; ++b) {
    const int c = __builtin_popcount(unsigned(b));
    for (int pc = 0; pc + c <= 16; ++pc) {
      uint32_t w[4];
      for (int d = 0; d < 4; ++d) w[d] = word[pc + 2 * d] | uint32_t(word[pc + 2 * d + 1]) << 16;
      const uint4 s0 = t.sel[2 * b], s1 = t.sel[2 * b + 1];
      const uint32_t lo[4] = {s0.x, s0.z, s1.x, s1.z}, hi[4] = {s0.y, s0.w, s1.y, s1.w};
      bool ok = true;
      uint16_t got[8];
      for (int d = 0; d < 4; ++d) {
        const uint32_t o = perm(w[1], w[0], lo[d], &ok) | perm(w[3], w[2], hi[d], &ok);
        got[2 * d] = uint16_t(o & 0xFFFF);
        got[2 * d + 1] = uint16_t(o >> 16);
      }
      for (int j = 0, r = 0; j < 8; ++j) {
        const uint16_t want = ((b >> j) & 1) ? word[pc + r++] : 0;
        if (got[j] != want) ok = false;
      }
      ++cases;
      if (!ok) {
        if (failures < 5) std::printf("byte %02x start %d wrong\n", b, pc);
        ++failures;
      }
    }
  }
  std::printf("expand bytes 256, cases %d, failures %d\n", cases, failures);
  return failures ? 1 : 0;
}
