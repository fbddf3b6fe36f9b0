// moe_layer_tb1.hip -- single-launch layer kernels for batches of 1 token.
#include "moe_layer.h"

namespace moe {
template const void* layer_fn<1>(int ns, int shape);
}  // namespace moe
