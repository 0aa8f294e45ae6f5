// q* split of the missed experts between PCIe copies and host compute.
//
// techfeed summary of "Meet FreeToken" (MarkTechPost), section "Bandwidth-adaptive
// execution (q* policy)": PCIe transfers and CPU expert execution both read host
// memory; with PCIe using B_P of the host bandwidth B_H, the CPU computes experts
// with the remaining B_H - B_P at the same time.  Of the m experts a step misses,
// about m * B_P / B_H are copied into the GPU cache and the others are computed
// on the CPU straight from host memory.
//
// Reading taken for the "about": each expert costs S bytes either way, so copying
// q takes q*S/B_P and computing m-q takes (m-q)*S/(B_H-B_P); the two run at once.
// The real balance point is m*B_P/B_H; the integer optimum is its floor or
// ceiling, whichever has the smaller makespan, with equal makespans going to the
// larger q (the copied expert also stays cached).
#include <algorithm>
#include <cmath>

#include "ecf_internal.h"

extern "C" int32_t qstar_split(int32_t m, double b_p, double b_h)
{
    if (m < 0 || std::isnan(b_p) || std::isnan(b_h) || !(b_h > 0.0))
        return ecf::set_error(ECF_EINVAL, "qstar_split: need m >= 0, b_h > 0, no NaN (m=%d b_p=%g b_h=%g)",
                              m, b_p, b_h);
    if (m == 0 || b_p <= 0.0)
        return 0;
    if (b_p >= b_h)
        return m;
    const double x = (double)m * b_p / b_h;
    const int32_t lo = std::min<int32_t>(m, (int32_t)std::floor(x));
    const int32_t hi = std::min<int32_t>(m, lo + 1);
    const double cpu_bw = b_h - b_p;
    const double t_lo = std::max(lo / b_p, (m - lo) / cpu_bw);
    const double t_hi = std::max(hi / b_p, (m - hi) / cpu_bw);
    return t_hi <= t_lo * (1.0 + 1e-12) ? hi : lo;
}
