// Diagonal-decay backward instantiations for f32 x/B/C/dy.
#include "bwd_launch.hpp"
#include "launch.hpp"

namespace ssd {
int run_bwd_diag_f32(const BwdArgs& a) {
    switch (a.P * 1000 + a.N) {
#define SSD_CASE(P, N) \
    case P * 1000 + N: return run_bwd_diag<float, P, N>(a);
        SSD_FOR_EACH_PN(SSD_CASE)
#undef SSD_CASE
        default: return 3;
    }
}
}  // namespace ssd
