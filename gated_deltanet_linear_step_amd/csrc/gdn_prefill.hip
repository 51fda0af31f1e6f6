// gdn_prefill.hip -- chunked prefill (placeholder until the chunk kernels land).
#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {

bool prefill_supported(int, int) { return false; }
size_t prefill_workspace_bytes(int, int, int, int, int64_t, int) { return 0; }
void prefill_carve(PrefillParams &, void *, int64_t) {}
hipError_t launch_prefill(const PrefillParams &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
