// moe_layer_tb2.hip -- single-launch layer kernels for batches of 2 tokens.
#include "moe_layer.h"

namespace moe {
template const void* layer_fn<2>(int ns, int shape);
}  // namespace moe
