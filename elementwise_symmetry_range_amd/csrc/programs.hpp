// programs.hpp -- the deployed polynomial programs (read-only data).
//
// Each entry is the program selected by the fitting workflow of "Fast
// Polynomial Transcendentals for LLMs" (arXiv 2610.00049), section 3.2:
// endpoint-constrained least squares on [0, Li] (Eqs. 7-8, 2,000 Chebyshev
// nodes, FP64), every coefficient rounded to BF16, replay in deployed order,
// maximum-error scoring on 8,000 points over [0, 12], Lc <= Li + 1, with the
// printed Table 2 bounds as a restriction.  coeff[j] is the BF16 bit pattern
// of the coefficient of t^j in the half-domain variable t = |x|.
//
//   sigmoid fwd D3  1/2 + sign(x) p(t^), clamp 5.28125 (Fig. 2's clamp)
//   tanh    fwd D4  sign(x) p(t^)
//   SiLU    fwd D3  x/2 + t p(t^), p = the sigmoid D3 polynomial (Eqs. 5-6)
//   GELU    fwd D5  x/2 + t p(t^), p fitted to Phi(t) - 1/2
//   sigmoid' D4     q(t^), direct derivative fit (even), c_0 = 1/4
//   tanh'    D4     q(t^), direct derivative fit (even), c_0 = 1
//   SiLU'    D3     1/2 + sign(x) q(t^), direct fit of s'(t) - 1/2 (odd, Eq. 9)
//   GELU'    D5     1/2 + sign(x) q(t^), the same construction for Phi + x phi
//
// The test suite re-derives every entry with an independent CPU fitter and
// checks the values returned by poly_program_info against it.
#pragma once
#include <cstdint>

namespace pa {

struct ProgramDef {
    int func;        // pa_func
    int deriv;       // 0 forward, 1 direct derivative
    int degree;
    float Li, Lc;
    uint16_t coeff[8];
};

constexpr ProgramDef kPrograms[] = {
    {1, 0, 3, 6.5f, 5.28125f, {0x0000, 0x3E90, 0xBD5B, 0x3B5D}},
    {2, 0, 4, 2.5f, 2.5f, {0x0000, 0x3F8B, 0xBEA5, 0xBCBD, 0x3C87}},
    {3, 0, 3, 6.5f, 5.28125f, {0x0000, 0x3E90, 0xBD5B, 0x3B5D}},
    {4, 0, 5, 3.75f, 2.75f, {0x0000, 0x3ECF, 0xBBEE, 0xBDA5, 0x3CDB, 0xBB2C}},
    {1, 1, 4, 4.75f, 4.75f, {0x3E80, 0xBB79, 0xBD8F, 0x3CB3, 0xBB00}},
    {2, 1, 4, 2.75f, 2.75f, {0x3F80, 0xBDE3, 0xBF65, 0x3F08, 0xBDB2}},
    {3, 1, 3, 3.75f, 4.25f, {0x0000, 0x3F17, 0xBE3E, 0x3C93}},
    {4, 1, 5, 4.25f, 2.75f, {0x0000, 0x3F6D, 0xBEB8, 0xBCD5, 0x3D05, 0xBB84}},
};

constexpr int kNumPrograms = sizeof(kPrograms) / sizeof(kPrograms[0]);

inline const ProgramDef *find_program(int func, int deriv)
{
    for (int i = 0; i < kNumPrograms; ++i)
        if (kPrograms[i].func == func && kPrograms[i].deriv == deriv) return &kPrograms[i];
    return nullptr;
}

}  // namespace pa
