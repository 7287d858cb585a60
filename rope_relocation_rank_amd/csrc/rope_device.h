// Device helpers shared by the gfx950 kernels (kernels.hip, attend.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kamera {

// cos and sin of phi = delta * omega, rounded to fp32.  phi is formed in fp64 and
// reduced by pi/2 with the two-constant Cody-Waite method (inside the FMA the first
// product is exact for |phi| < 2^53); on the reduced |r| <= pi/4 the Taylor series of
// sin (through r^11) and cos (through r^12) are summed in fp64, whose truncation error
// (< 2e-9 relative) stays far below fp32 rounding; the quadrant picks signs and order.
__device__ __forceinline__ float2 phase_of(double omega, int64_t delta) {
  const double kPio2a = 0x1.921fb54442d18p+0;    // pi/2 rounded to a double
  const double kPio2b = 0x1.1a62633145c07p-54;   // pi/2 minus the above
  const double kTwoOverPi = 0x1.45f306dc9c883p-1;
  const double phi = (double)delta * omega;
  const double k = rint(phi * kTwoOverPi);
  double r = fma(-k, kPio2a, phi);
  r = fma(-k, kPio2b, r);
  const double r2 = r * r;
  double sp = -1.0 / 39916800.0;
  sp = fma(sp, r2, 1.0 / 362880.0);
  sp = fma(sp, r2, -1.0 / 5040.0);
  sp = fma(sp, r2, 1.0 / 120.0);
  sp = fma(sp, r2, -1.0 / 6.0);
  const double sr = fma(r * r2, sp, r);
  double cp = 1.0 / 479001600.0;
  cp = fma(cp, r2, -1.0 / 3628800.0);
  cp = fma(cp, r2, 1.0 / 40320.0);
  cp = fma(cp, r2, -1.0 / 720.0);
  cp = fma(cp, r2, 1.0 / 24.0);
  cp = fma(cp, r2, -0.5);
  const double cr = fma(r2, cp, 1.0);
  const int qd = (int)((int64_t)k & 3);
  const double c = qd == 0 ? cr : qd == 1 ? -sr : qd == 2 ? -cr : sr;
  const double s = qd == 0 ? sr : qd == 1 ? cr : qd == 2 ? -sr : -cr;
  return make_float2((float)c, (float)s);
}

// Value of lane (l ^ X) within each 16-lane row (X in {1, 2, 4, 8}) or 32-lane half
// (X = 16).  Every lane of the wavefront must execute it.
template <int X>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (X == 1)  // quad_perm [1,0,3,2]
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);
  else if constexpr (X == 2)  // quad_perm [2,3,0,1]
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);
  else if constexpr (X == 8)  // row_ror:8 swaps the two 8-lane halves of a row
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, true);
  else if constexpr (X == 4)  // swizzle bit mode: and 0x1f, or 0, xor 4
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
  else  // swizzle bit mode: and 0x1f, or 0, xor 16
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

}  // namespace kamera
