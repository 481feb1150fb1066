// KV-major prefill attention (work in progress): not yet available.
#include "launch.hpp"

namespace msa {

size_t kvmajor_workspace_bytes(const Dims &) { return 0; }

hipError_t launch_attn_kvmajor_bf16(const Dims &, const uint16_t *, const uint16_t *,
                                    const uint16_t *, const int32_t *, uint16_t *, float *, void *,
                                    hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace msa
