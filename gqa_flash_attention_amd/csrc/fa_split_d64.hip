// Split-KV kernels for head dim (tile width) 64.
#include "fa_split.h"

namespace gqafa {

hipError_t launch_split_d64(const SplitDesc& d, hipStream_t stream) { return run_split_d<64>(d, stream); }

}  // namespace gqafa
