// Paged prefill / append attention for bf16.
// Interim: routes to the row kernel until the MFMA tile kernel lands.
#include "internal.h"

namespace pkv {

hipError_t launch_prefill_mfma(int32_t head_dim, int32_t group, const AttnArgs& a, hipStream_t st,
                               bool* supported) {
  return launch_attn_rows(kBF16, head_dim, group, a, st, supported);
}

}  // namespace pkv
