// Split-KV kernels for head dim (tile width) 256.
#include "fa_split.h"

namespace gqafa {

hipError_t launch_split_d256(const SplitDesc& d, hipStream_t stream) { return run_split_d<256>(d, stream); }

}  // namespace gqafa
