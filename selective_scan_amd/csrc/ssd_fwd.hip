// Mamba-2 SSD chunked scan on gfx950 (placeholder until the chunked kernel lands).
#include "common.h"
#include "launch.h"

namespace ssm {

const char* ssd_unsupported_reason(int, int, int, int, int, bool) {
    return "the SSD kernel is not built in this version";
}

size_t ssd_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_ssd_fwd(const SsdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssm
