// Kernel instances of one GQA group size G (set with -DSSPEC_G=<G>), so that
// the eight groups compile in parallel.
#include "kernel.hpp"

#ifndef SSPEC_G
#error "compile with -DSSPEC_G=<1..8>"
#endif

namespace sspec {

#define SSPEC_CAT2(a, b) a##b
#define SSPEC_CAT(a, b) SSPEC_CAT2(a, b)
// SSPEC_ONLY_G (development builds only) leaves the other groups' rows empty
const char* SSPEC_CAT(build_config_g, SSPEC_G)() { return build_config(); }
#if defined(SSPEC_ONLY_G) && SSPEC_ONLY_G != 0 && SSPEC_ONLY_G != SSPEC_G
std::array<KernelFn, 8> SSPEC_CAT(kernel_table_g, SSPEC_G)() { return {}; }
#else
std::array<KernelFn, 8> SSPEC_CAT(kernel_table_g, SSPEC_G)() { return kernel_row<SSPEC_G>(); }
#endif

}  // namespace sspec
