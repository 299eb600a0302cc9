// Discretisation variants of the Mamba-1 selective scan on gfx950: exact
// zero-order hold ("Efficient Sequence Modeling: From S4 to Mamba-3", section 04
// "Math-verified discretization" and Q01) and Delta = softplus(delta + bias)
// computed in the kernel. The kernels are the plain scan's (scan_core.h) with
// the variant selected by their template parameter V.
#include "scan_core.h"

namespace ssm {

bool scan_var_supported_n(int N) {
    return N == 4 || N == 8 || N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
}

namespace {
template <bool BF16, int V>
hipError_t var_n(const ScanArgs& a, hipStream_t st) {
    switch (a.N) {
        case 4: return launch_n<4, BF16, V>(a, st);
        case 8: return launch_n<8, BF16, V>(a, st);
        case 16: return launch_n<16, BF16, V>(a, st);
        case 32: return launch_n<32, BF16, V>(a, st);
        case 64:
        case 128:
        case 256: return launch_n<kChunkN, BF16, V>(a, st);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_scan_fwd_var(const ScanArgs& a, hipStream_t st) {
    if (a.disc == 1) return a.bf16 ? var_n<true, 2>(a, st) : var_n<false, 2>(a, st);
    return a.bf16 ? var_n<true, 1>(a, st) : var_n<false, 1>(a, st);
}

}  // namespace ssm
