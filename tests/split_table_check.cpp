// Host check of the split tables of the 4:8 / 8:16 products (nm_prefill_impl.h).
// For every 16-bit mask chunk that a 4:8 or 8:16 row can hold (every choice of 4 of each 8
// columns, every choice of 8 of 16 columns) and 8 distinct nonzero values, the two 2:4
// operands built from the table entries, decoded as the sparse matrix instruction reads
// them (nibble g of the index word = positions p0 | p1 << 2 of group g's two halves), must
// add up to the dense 16 columns: the kept values in ascending column order, zeros elsewhere,
// with no position written twice. The byte selection of v_perm_b32 is emulated from its
// definition (selector bytes 0..3 pick bytes of the second source, 4..7 of the first, 12 a
// zero byte).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "nm_prefill_impl.h"

using nm::prefill_detail::SplitTable;

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

static int check(const SplitTable& t, uint32_t m16) {
  uint16_t v[8];
  for (int i = 0; i < 8; ++i) v[i] = uint16_t(0x3C00 + 17 * i + 1);   // distinct, nonzero
  const uint32_t d[4] = {v[0] | uint32_t(v[1]) << 16, v[2] | uint32_t(v[3]) << 16,
                         v[4] | uint32_t(v[5]) << 16, v[6] | uint32_t(v[7]) << 16};
  uint32_t want[16] = {0};
  for (int c = 0, r = 0; c < 16; ++c)
    if ((m16 >> c) & 1) want[c] = v[r++];
  const int e0 = int(m16 & 0xFF), e1 = 256 + int(m16 >> 8);
  const uint4 s[4] = {t.sel[2 * e0], t.sel[2 * e0 + 1], t.sel[2 * e1], t.sel[2 * e1 + 1]};
  bool ok = true;
  auto pick = [&](uint32_t lo, uint32_t hi) { return perm(d[1], d[0], lo, &ok) | perm(d[3], d[2], hi, &ok); };
  const uint32_t A[4] = {pick(s[0].x, s[0].y), pick(s[1].x, s[1].y), pick(s[2].x, s[2].y), pick(s[3].x, s[3].y)};
  const uint32_t B[4] = {pick(s[0].z, s[0].w), pick(s[1].z, s[1].w), pick(s[2].z, s[2].w), pick(s[3].z, s[3].w)};
  const uint32_t i0 = t.idx[e0], i1 = t.idx[e1];
  const uint32_t ia = perm(i1, i0, 0x0C0C0400u, &ok), ib = perm(i1, i0, 0x0C0C0501u, &ok);
  uint32_t got[16] = {0};
  for (int op = 0; op < 2; ++op) {
    const uint32_t* X = op ? B : A;
    const uint32_t ix = op ? ib : ia;
    for (int g = 0; g < 4; ++g) {
      const unsigned code = (ix >> (4 * g)) & 15, p0 = code & 3, p1 = code >> 2;
      if (!(p0 < p1)) ok = false;
      const uint32_t h[2] = {X[g] & 0xFFFF, X[g] >> 16};
      const unsigned pos[2] = {4 * g + p0, 4 * g + p1};
      for (int k = 0; k < 2; ++k) {
        if (!h[k]) continue;
        if (got[pos[k]]) ok = false;
        got[pos[k]] = h[k];
      }
    }
  }
  for (int c = 0; c < 16; ++c) ok = ok && got[c] == want[c];
  if (!ok) std::printf("FAIL mask %04x\n", m16);
  return ok ? 0 : 1;
}

int main() {
  static const SplitTable t = nm::prefill_detail::make_split_table();
  int fails = 0, n48 = 0, n816 = 0;
  for (uint32_t m16 = 0; m16 < 65536; ++m16) {
    const bool p48 = __builtin_popcount(m16 & 0xFF) == 4 && __builtin_popcount(m16 >> 8) == 4;
    const bool p816 = __builtin_popcount(m16) == 8;
    if (p48) ++n48;
    if (p816) ++n816;
    if (p48 || p816) fails += check(t, m16);
  }
  std::printf("4:8 chunks %d, 8:16 chunks %d, failures %d\n", n48, n816, fails);
  return fails == 0 && n48 == 4900 && n816 == 12870 ? 0 : 1;
}
