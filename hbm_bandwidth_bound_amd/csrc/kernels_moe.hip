// kernels_moe.hip -- instantiation of the decode and prompt kernels for mixture-of-experts
// layers: head_dim 128 with 8 query heads per KV head.
#include "monokernel_impl.h"

namespace kie {

KernelFn kernel_moe(int G, int HD, bool prompt) {
  if (G == 8 && HD == 128) return prompt ? kie_moe_prompt_kernel<8, 128> : kie_moe_decode_kernel<8, 128>;
  return nullptr;
}

}  // namespace kie
