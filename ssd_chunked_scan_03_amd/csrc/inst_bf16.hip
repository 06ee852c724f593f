// Kernel instantiations for bfloat16 x/B/C/y.
#include "launch.hpp"

namespace ssd {
int run_bf16(const RunArgs& a) {
    switch (a.P * 1000 + a.N) {
#define SSD_CASE(P, N) \
    case P * 1000 + N: return run<bf16, P, N>(a);
        SSD_FOR_EACH_PN(SSD_CASE)
#undef SSD_CASE
        default: return 3;
    }
}
}  // namespace ssd
