// kernels_hd64.hip -- instantiations of the decode and prompt kernels for head_dim 64.
#include "monokernel_impl.h"

namespace kie {

KernelFn kernel_hd64(int G, bool prompt) {
  switch (G) {
    case 1: return prompt ? kie_prompt_kernel<1, 64> : kie_decode_kernel<1, 64>;
    case 2: return prompt ? kie_prompt_kernel<2, 64> : kie_decode_kernel<2, 64>;
    case 4: return prompt ? kie_prompt_kernel<4, 64> : kie_decode_kernel<4, 64>;
    case 8: return prompt ? kie_prompt_kernel<8, 64> : kie_decode_kernel<8, 64>;
    default: return nullptr;
  }
}

}  // namespace kie
