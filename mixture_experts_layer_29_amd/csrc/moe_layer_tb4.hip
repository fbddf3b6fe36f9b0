// moe_layer_tb4.hip -- single-launch layer kernels for batches of 3 or 4 tokens.
#include "moe_layer.h"

namespace moe {
template const void* layer_fn<4>(int ns, int shape);
}  // namespace moe
