/*
 * quotient_exactness.c -- host-side exhaustive check of the division step of
 * the library's fp8 quantisation (the bf16 / fp16 value divided by a per-layer
 * or per-tensor fp32 dequantisation scale s, which "PR #55356 完整报告",
 * 关键源码片段, applies through scaled_convert, and which "PR #51772 完整报告",
 * 实现拆解 item 1, requires to give codes bit-identical to torch's cast).
 *
 * The GPU kernels do not divide.  With r = RN(1/s) computed once they take
 *   q0 = RN(x * r)            (within one ulp of x / s)
 *   e  = RN(fma(-q0, s, x))   (the exact remainder x - q0 * s)
 *   q  = RN(fma(e, r, q0))
 * and rely on q being the IEEE binary32 quotient RN(x / s) (Markstein's
 * correction step).  This program evaluates the same sequence with the same
 * binary32 operations on the host (built with -ffp-contract=off, so that
 * x * r is its own rounded product; fmaf is the correctly rounded fused
 * multiply-add) and compares q with x / s bit for bit.
 *
 * Sweep "sig16 B": every significand of a 16-bit source format with B
 * fraction bits (7 for bf16, 10 for fp16) against every fp32 significand of
 * s, both in [1, 2).  Multiplying x by 2^a and s by 2^b scales r, q0, e and
 * q by powers of two exactly, so while no intermediate leaves the normal
 * range this covers every normal x and s.
 *
 * Sweep "edges": every finite bf16 pattern x (subnormals and zeros
 * included) against scales of every binary32 exponent, subnormal ones
 * included, each with 24 significands (1.0, the largest, and 22 fixed
 * pseudo-random ones).  A pair counts as a disagreement only where the
 * difference can reach an fp8 code: q and x / s differ in bits, and not
 * (a) both magnitudes are below 2^-18 (both round to a zero code in e4m3fn
 * and e5m2), nor (b) both are at least 2^17 or NaN / Inf (both saturate,
 * since the kernels clamp with med3 and rewrite the sign).  The program
 * prints, per exponent of s, the number of disagreements, so that the range
 * of scales for which the quantisation is exact can be stated.
 *
 * Sweep "bf16-uncorrected" repeats the bf16 significand sweep with q = q0
 * (the correction step left out), a planted mistake that must show.
 *
 * Output: one line per sweep, "sig16 B mismatches N" or
 * "edges exp E mismatches N" for every exponent E of s with N > 0, then
 * "edges total N".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t u_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float markstein_quotient(float x, float s, float r) {
  const float q0 = x * r;
  const float e = fmaf(-q0, s, x);
  return fmaf(e, r, q0);
}

/* uncorrected = 1 drops the correction step (q = q0): a planted mistake the
 * sweep must catch. */
static long long sweep_significands(int frac_bits, int uncorrected) {
  long long bad = 0;
  const int nx = 1 << frac_bits;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 1)
  for (int mx = 0; mx < nx; ++mx) {
    const float x = f_of(0x3F800000u | ((uint32_t)mx << (23 - frac_bits)));
    for (uint32_t fs = 0; fs < (1u << 23); ++fs) {
      const float s = f_of(0x3F800000u | fs);
      const float r = 1.0f / s;
      const float q = uncorrected ? x * r : markstein_quotient(x, s, r);
      if (u_of(q) != u_of(x / s)) ++bad;
    }
  }
  return bad;
}

/* does a quotient difference reach an fp8 code? (see the header) */
static int differs_for_fp8(float q, float ref) {
  if (u_of(q) == u_of(ref)) return 0;
  const float aq = fabsf(q), ar = fabsf(ref);
  if (aq < 0x1p-18f && ar < 0x1p-18f) return 0;
  const int big_q = !(aq < 0x1p17f);   /* also NaN */
  const int big_r = !(ar < 0x1p17f);
  if (big_q && big_r) return 0;
  return 1;
}

static long long sweep_edges(void) {
  enum { NSIG = 24 };
  uint32_t sig[NSIG];
  sig[0] = 0;
  sig[1] = 0x7FFFFFu;
  uint64_t z = 0x9E3779B97F4A7C15ull;
  for (int i = 2; i < NSIG; ++i) {
    z ^= z << 13;
    z ^= z >> 7;
    z ^= z << 17;
    sig[i] = (uint32_t)(z >> 20) & 0x7FFFFFu;
  }
  long long per_exp[256];
  memset(per_exp, 0, sizeof per_exp);
#pragma omp parallel for schedule(dynamic, 1)
  for (int be = 0; be < 255; ++be) {
    long long bad = 0;
    for (int k = 0; k < NSIG; ++k) {
      const uint32_t su = ((uint32_t)be << 23) | sig[k];
      if (su == 0) continue; /* s = 0 is not a scale */
      const float s = f_of(su);
      const float r = 1.0f / s;
      for (uint32_t b = 0; b < 65536u; ++b) {
        if ((b & 0x7F80u) == 0x7F80u) continue; /* Inf / NaN inputs are patched apart */
        const float x = f_of(b << 16);
        if (differs_for_fp8(markstein_quotient(x, s, r), x / s)) ++bad;
      }
    }
    per_exp[be] = bad;
  }
  long long total = 0;
  for (int be = 0; be < 255; ++be) {
    if (per_exp[be]) printf("edges exp %d mismatches %lld\n", be - 127, per_exp[be]);
    total += per_exp[be];
  }
  printf("edges total %lld\n", total);
  return total;
}

int main(int argc, char** argv) {
  int done = 0;
  for (int i = 1; i < argc; ++i) {
    if (!strcmp(argv[i], "bf16")) {
      printf("sig16 7 mismatches %lld\n", sweep_significands(7, 0));
      done = 1;
    } else if (!strcmp(argv[i], "fp16")) {
      printf("sig16 10 mismatches %lld\n", sweep_significands(10, 0));
      done = 1;
    } else if (!strcmp(argv[i], "bf16-uncorrected")) {
      printf("sig16 7 uncorrected mismatches %lld\n", sweep_significands(7, 1));
      done = 1;
    } else if (!strcmp(argv[i], "edges")) {
      sweep_edges();
      done = 1;
    } else {
      fprintf(stderr, "unknown sweep %s\n", argv[i]);
      return 2;
    }
  }
  if (!done) {
    fprintf(stderr, "usage: %s bf16|fp16|bf16-uncorrected|edges ...\n", argv[0]);
    return 2;
  }
  return 0;
}
