// Host stand-ins for the device-side launchers and workspace sizes of
// libmf.so, so that the C-ABI layer (abi.cpp) can be built for the host
// alone under AddressSanitizer / UndefinedBehaviorSanitizer.  Every launcher
// counts its call and fails, as a launch would on a machine without a GPU.
#include <hip/hip_runtime.h>

#include "mf_internal.h"

long g_launches = 0;

namespace mf {

static hipError_t counted() {
    ++g_launches;
    return hipErrorNoDevice;
}

size_t attn_workspace_bytes(int32_t n_seq, int64_t, int32_t, int32_t) {
    return 4096 + 16 * size_t(n_seq > 0 ? n_seq : 0);
}
size_t attn_bwd_workspace_bytes(int32_t n_seq, int64_t T, int32_t, int32_t) {
    return 4096 + 16 * size_t(n_seq > 0 ? n_seq : 0) + size_t(T > 0 && T < (1 << 20) ? T : 0);
}
size_t block_qkv_workspace_bytes(int64_t T, int32_t C, int32_t D) {
    return T > 0 && C > 0 && T < (1 << 20) && C < (1 << 16) ? size_t(T) * size_t(C) * 2 + size_t(T) * size_t(D > 0 ? D : 0) * 4
                                                             : 256;
}
size_t causal_attn_workspace_bytes(int32_t n_seq, int64_t) { return 256 + 16 * size_t(n_seq > 0 ? n_seq : 0); }
size_t elementwise_bwd_workspace_bytes(int64_t T, int32_t C, int32_t n) {
    return T > 0 && C > 0 && T < (1 << 20) && C < (1 << 16) ? size_t(T / 4 + 1) * size_t(C) * size_t(n) * 4 : 256;
}

hipError_t launch_modulate_rope(const ModRopeArgs&, hipStream_t) { return counted(); }
hipError_t launch_modulate_rope_bwd(const ModRopeBwdArgs&, hipStream_t) { return counted(); }
hipError_t launch_gated_residual_bwd(const GatedResBwdArgs&, hipStream_t) { return counted(); }
hipError_t launch_gated_residual(const GatedResArgs&, hipStream_t) { return counted(); }
hipError_t launch_varlen_attn_fwd(const AttnArgs&, hipStream_t) { return counted(); }
hipError_t launch_varlen_attn_fwd_noalloc(const AttnArgs&, hipStream_t) { return counted(); }
hipError_t launch_varlen_attn_bwd(const AttnBwdArgs&, hipStream_t) { return counted(); }
hipError_t launch_block_qkv(const BlockQkvArgs&, hipStream_t) { return counted(); }
hipError_t launch_block_out(const BlockOutArgs&, hipStream_t) { return counted(); }
hipError_t launch_cfg_euler(const CfgEulerArgs&, hipStream_t) { return counted(); }
hipError_t launch_qk_norm_rope(const QkNormRopeArgs&, hipStream_t) { return counted(); }
hipError_t launch_varlen_attn_causal(const CausalAttnArgs&, hipStream_t) { return counted(); }
void set_attn_fwd_grid(int) {}

}  // namespace mf
