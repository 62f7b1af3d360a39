// Split-KV kernels for head dim (tile width) 128.
#include "fa_split.h"

namespace gqafa {

hipError_t launch_split_d128(const SplitDesc& d, hipStream_t stream) { return run_split_d<128>(d, stream); }

}  // namespace gqafa
