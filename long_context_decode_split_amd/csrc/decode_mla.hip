// Split-KV decode attention for MLA caches (one latent KV head, Dk = 576,
// Dv = 512, V = the first 512 columns of each latent row).
#include "hx_common.h"

namespace hx {

hipError_t launch_mla_partial(const PartialArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace hx
