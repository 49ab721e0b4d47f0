// Exhaustive host check of the cache-append kernel's arithmetic (CPU only):
// the kernel source itself is included, so the quotient checked is the
// kernel's own.
//  (1) The emulator's model of the fp32 -> e4m3 conversion (which the emulated
//      parity tests run) equals a plain encoder that rounds the fp32 mantissa
//      to 3 bits with ties to even (k * 2^-9 steps below 2^-6), on every 97th
//      fp32 value in [-448, 448] and around every code and every midpoint.  The GPU check in tests/gpu_checks compares the
//      hardware conversion with the same plain encoder.
//  (2) For every bf16 value m > 0 taken as a row's max|x| with scale
//      s = m / 448 >= 2^-64, and every bf16 value a <= m, the quotient of the
//      reciprocal + correction path gives the same code as the correctly
//      rounded a / s.
// Exit status 0 when both hold.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "append_kernel.hip"

using namespace mla;

static float u2f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

static uint32_t plain_encoder(float a) {
  if (a < 0.015625f) return uint32_t(std::nearbyint(a * 512.f));
  const uint32_t v = f2u(a), m = v & 0x7FFFFFu;
  uint32_t code = (((v >> 23) - 120u) << 3) | (m >> 20);
  const uint32_t rest = m & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ++code;
  return code;
}

static float plain_value(uint32_t c) {   // value of a non-negative code
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? std::ldexp(float(m), -9) : std::ldexp(float(8 + m), int(e) - 10);
}

int main() {
  uint64_t bad1 = 0, n1 = 0;
  auto check1 = [&](float f) {
    ++n1;
    const uint32_t want = plain_encoder(f);
    if ((emu::e4m3_rne(f) != want || emu::e4m3_rne(-f) != (want | 0x80u)) && bad1++ < 5)
      std::printf("encoder differs at %08x\n", f2u(f));
  };
  // every 97th fp32 pattern in [0, 448], and around every code and midpoint
  for (uint32_t u = 0; u <= f2u(448.f); u += 97) check1(u2f(u));
  for (uint32_t c = 0; c < 126; ++c) {
    const float v0 = plain_value(c), v1 = plain_value(c + 1), mid = 0.5f * (v0 + v1);
    for (float f : {v0, mid, v1})
      for (float g : {std::nextafter(f, 0.f), f, std::nextafter(f, 449.f)})
        if (g <= 448.f) check1(g);
  }
  std::printf("encoder: %llu values, %llu differ\n", (unsigned long long)n1,
              (unsigned long long)bad1);
  uint64_t bad2 = 0, n2 = 0;
  const float thr = std::ldexp(1.f, -64);
  for (uint32_t mb = 1; mb < 0x7F80u; ++mb) {
    const float s = u2f(mb << 16) / 448.f;
    if (!(s >= thr)) continue;
    const float y = 1.f / s;
    for (uint32_t ab = 0; ab <= mb; ++ab, ++n2) {
      const float a = u2f(ab << 16);
      const uint32_t want = plain_encoder(std::fmin(a / s, 448.f));
      const uint32_t got = plain_encoder(std::fmin(quotient(a, s, y, false), 448.f));
      if (want != got && bad2++ < 5) std::printf("code differs: max %08x, a %08x\n", mb << 16, ab << 16);
    }
  }
  std::printf("division: %llu pairs, %llu codes differ\n", (unsigned long long)n2,
              (unsigned long long)bad2);
  return (bad1 || bad2) ? 1 : 0;
}
