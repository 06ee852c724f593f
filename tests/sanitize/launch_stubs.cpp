// Stand-ins for the library's launch sequences, for the host-code sanitizer build: that
// build links the C ABI unit alone (its checks, layouts and status strings), and every
// call the check program makes is refused before any launch, so reaching one of these
// is itself a failure.
#include <cstdio>
#include <cstdlib>

namespace ssd {
struct RunArgs;
struct BwdArgs;
[[noreturn]] static void reached(const char* what) {
    std::fprintf(stderr, "launch sequence %s reached: a call was not refused on the host\n", what);
    std::abort();
}
int run_bf16(const RunArgs&) { reached("run_bf16"); }
int run_f32(const RunArgs&) { reached("run_f32"); }
int run_bwd_bf16(const BwdArgs&) { reached("run_bwd_bf16"); }
int run_bwd_f32(const BwdArgs&) { reached("run_bwd_f32"); }
int run_bwd_diag_bf16(const BwdArgs&) { reached("run_bwd_diag_bf16"); }
int run_bwd_diag_f32(const BwdArgs&) { reached("run_bwd_diag_f32"); }
}  // namespace ssd
