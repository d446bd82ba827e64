// Kernel-launch table of the host-only sanitizer build of the C ABI layer.
// Test infrastructure: the CPU tests link api.cpp and order.cpp against these
// stubs (compiled with g++ -fsanitize=address,undefined, no device code) and
// drive the validation, cache layout, schedule and Hilbert-order paths.  Every
// stub refuses to launch, so this build can never return a result that was
// not computed: a call that gets past validation fails with RT_E_LAUNCH (or
// RT_E_DEVICE, as there is no GPU where the sanitizer build runs).
#include "../../sparse_attention_diffusion_amd/csrc/internal.h"

namespace rettn {

hipError_t launch_permute(const PermuteArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bf16(AttnMode, int, const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_f32(AttnMode, int, const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_select(bool, int, const SelectArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t select_scratch(void**) { return hipErrorNoDevice; }

}  // namespace rettn
