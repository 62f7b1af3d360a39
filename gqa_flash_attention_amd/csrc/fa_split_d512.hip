// Split-KV kernels for head dim (tile width) 512.
#include "fa_split.h"

namespace gqafa {

hipError_t launch_split_d512(const SplitDesc& d, hipStream_t stream) { return run_split_d<512>(d, stream); }

}  // namespace gqafa
