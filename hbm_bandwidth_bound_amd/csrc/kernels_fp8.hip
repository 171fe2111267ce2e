// kernels_fp8.hip -- instantiations of the decode and prompt kernels for 8-bit (e4m3fn) weights:
// head_dim 64 or 128 with 2 or 4 query heads per KV head.
#include "monokernel_impl.h"

namespace kie {

KernelFn kernel_fp8(int G, int HD, bool prompt) {
  if (HD == 64 && G == 2) return prompt ? kie_fp8_prompt_kernel<2, 64> : kie_fp8_decode_kernel<2, 64>;
  if (HD == 128 && G == 2) return prompt ? kie_fp8_prompt_kernel<2, 128> : kie_fp8_decode_kernel<2, 128>;
  if (HD == 128 && G == 4) return prompt ? kie_fp8_prompt_kernel<4, 128> : kie_fp8_decode_kernel<4, 128>;
  return nullptr;
}

}  // namespace kie
