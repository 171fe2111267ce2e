// monokernel.hip -- kernel selection and LDS sizing for the decode monokernel (the device code
// is in monokernel_impl.h; its instantiations are in kernels_hd64.hip, kernels_hd128.hip,
// kernels_moe.hip and kernels_fp8.hip).
#include "monokernel_impl.h"

namespace kie {

KernelFn kernel_hd64(int G, bool prompt);
KernelFn kernel_hd128(int G, bool prompt);
KernelFn kernel_moe(int G, int HD, bool prompt);
KernelFn kernel_fp8(int G, int HD, bool prompt);

int32_t lds_bytes_for(const Shape& s) { return lds_bytes_for_impl(s); }
int32_t lds_slot_offset(const Shape& s) { return xb_fits(s) ? lds_base_bytes(s) : 0; }
int32_t topk_capacity_floats(const Shape& s) { return merge_floats(s); }

KernelFn decode_kernel_for(int G, int HD, bool prompt, bool moe, bool w8) {
  if (moe) return w8 ? nullptr : kernel_moe(G, HD, prompt);
  if (w8) return kernel_fp8(G, HD, prompt);
  if (HD == 128) return kernel_hd128(G, prompt);
  if (HD == 64) return kernel_hd64(G, prompt);
  return nullptr;
}

}  // namespace kie
