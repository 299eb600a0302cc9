// Mamba-1 selective scan on gfx950, exponential-Euler with Delta as given: the
// host side of ssm_scan_fwd (kernels in scan_core.h).
#include "scan_core.h"

namespace ssm {
bool scan_supported_n(int N) {
    return N == 4 || N == 8 || N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
}

ScanPlan scan_plan(int B, int L, int D, int N) {
    const Geom g = geom(B, L, D, N);
    return ScanPlan{g.S, g.Ls};
}

size_t scan_workspace_bytes(int B, int L, int D, int N) {
    const Geom g = geom(B, L, D, N);
    // a short chain run in one workgroup needs none
    if (fused_call(g, B, D, N)) return 0;
    // one workgroup holds every state chunk (N <= 128) and finishes y itself; a
    // single segment needs no carries
    if (sink_planes(N) == 1) return g.S <= 1 ? 0 : ws_layout(B, D, N, g.S, g.G).total * sizeof(float);
    // else the summed C . h of each group of state chunks follows the carry arrays (YP)
    return (ws_layout(B, D, N, g.S, g.G).total + (size_t)sink_planes(N) * B * L * D) * sizeof(float);
}

hipError_t launch_scan_fwd(const ScanArgs& a, hipStream_t st) {
    return a.bf16 ? launch_dtype<true>(a, st) : launch_dtype<false>(a, st);
}

}  // namespace ssm
