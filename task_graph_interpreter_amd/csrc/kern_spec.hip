// One specialisation of the decode kernels, selected at compile time with
// -DMK_SPEC_FN=<ks_name> -DMK_SPEC_ARGS=<weights bf16>,<cache bf16>,<batch rows>,
// <kblocks hidden>,<kblocks intermediate> (the build compiles this file once per
// entry of specs.def).
#include "kernels.h"

#if !defined(MK_SPEC_FN) || !defined(MK_SPEC_ARGS)
#error "compile with -DMK_SPEC_FN=... -DMK_SPEC_ARGS=..."
#endif

namespace mk {
KernelSet MK_SPEC_FN() { return kernel_set<Spec<MK_SPEC_ARGS>>(); }
}  // namespace mk
