// kernels_hd128.hip -- instantiations of the decode and prompt kernels for head_dim 128.
#include "monokernel_impl.h"

namespace kie {

KernelFn kernel_hd128(int G, bool prompt) {
  switch (G) {
    case 1: return prompt ? kie_prompt_kernel<1, 128> : kie_decode_kernel<1, 128>;
    case 2: return prompt ? kie_prompt_kernel<2, 128> : kie_decode_kernel<2, 128>;
    case 4: return prompt ? kie_prompt_kernel<4, 128> : kie_decode_kernel<4, 128>;
    case 8: return prompt ? kie_prompt_kernel<8, 128> : kie_decode_kernel<8, 128>;
    default: return nullptr;
  }
}

}  // namespace kie
