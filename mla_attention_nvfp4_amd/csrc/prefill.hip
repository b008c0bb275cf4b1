// Varlen causal MLA prefill with NVFP4 fake quantization and fused NVFP4
// output (gfx950).  Placeholder until the kernel lands: reports "not
// supported" so the C ABI returns MLA_ERR_UNSUPPORTED.
#include "launch.hpp"

namespace mla {

size_t prefill_workspace_bytes(int64_t, int, unsigned) { return 0; }

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
