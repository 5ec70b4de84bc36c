// attn_programs.hpp -- the sigmoid-attention program (read-only data).
#pragma once
#include <cstdint>

namespace pa {

// Sigmoid attention (section 3.4, section 5.2.3, Eq. 14): P = sigma(s - ln n)
// for scores s = q.k / sqrt(D), as one cubic per region on the clamped score,
// with ln n and the 1/n scaling folded into the coefficients; valid for the
// one sequence length n it was fitted for.  The BF16 constants are the ones
// Appendix C's Listings 1-2 print.  Region 1 when x >= thr.  Derivative
// surrogate P~(x) (a + b x) (the factored D4 of section 3.4).
struct SigmoidAttnDef {
    int n;
    uint16_t thr, lo, hi;
    uint16_t c[2][4];    // c[r][j]: coefficient of x^j in region r
    uint16_t a[2], b[2];
};

constexpr SigmoidAttnDef kSigmoidAttn = {
    4096, 0x3FA0, 0xC0C0, 0x40C0,
    {{0x3980, 0x3987, 0x3909, 0x37E8}, {0xBB09, 0x3B8C, 0xBB11, 0x3A09}},
    {0x3F80, 0x3F81},
    {0xBC10, 0xBB38},
};

}  // namespace pa
