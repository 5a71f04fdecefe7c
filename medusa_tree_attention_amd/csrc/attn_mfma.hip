// Matrix-core tree attention (bf16, d_h = 128) -- not enabled yet; the
// wavefront-per-row path serves every shape until it is.

#include "attn_common.h"

namespace medusa {

bool mfma_path_applies(medusa_dtype, int32_t, int32_t, int32_t, int32_t) { return false; }

size_t attn_workspace_bytes(medusa_dtype, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) {
  return 4096;
}

medusa_status run_mfma(AttnArgs&, hipStream_t, void*, void*) { return MEDUSA_EUNSUPPORTED; }

}  // namespace medusa
