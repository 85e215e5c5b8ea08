// Packed classifier-free guidance + Euler sampler step after the last block
// (gfx950).
//
// The backbone predicts a velocity for the straight interpolation
// z_t = (1 - t) z + t eps between data and noise (gist.science "Resumo
// Tecnico: Mage-Flow", Metodologia; picx.dev summary, Introduction and
// Theoretical Foundation); the conditional and unconditional branches run
// packed in one forward (picx.dev, Methodology > Native-Resolution MMDiT), and
// the Turbo variants sample in 4 steps.  Per evolving latent token k with
// packed rows (rc, ru) of its two copies and every latent channel:
//   v      = v[ru] + w (v[rc] - v[ru])          (fp32 from the bf16 velocities)
//   z'[k]  = z[k] + (t - t_next) v              (fp32 sampler state)
//   x[rc] = x[ru] = bf16(z'[k])                 (the next forward's input rows)
//
// HBM-bound: one thread per 8 channels of a token (16-byte bf16 loads and
// stores, 32-byte fp32 loads and stores), 64-bit row indices never needed.
#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

__global__ __launch_bounds__(256) void cfg_euler_kernel(CfgEulerArgs a) {
    const int chunks = a.Cl >> 3;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= a.N * chunks) return;
    const int64_t k = i / chunks;
    const int c8 = int(i - k * chunks) * 8;
    const int2 r = reinterpret_cast<const int2*>(a.rows)[k];
    float vc[8], vu[8];
    unpack8(ld16(a.v + int64_t(r.x) * a.ld_v + c8), vc);
    unpack8(ld16(a.v + int64_t(r.y) * a.ld_v + c8), vu);
    const f32x4_t* zp = reinterpret_cast<const f32x4_t*>(a.z + k * a.Cl + c8);
    const f32x4_t z0 = zp[0], z1 = zp[1];
    const float dt = a.t - a.t_next;
    float zn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float g = vu[j] + a.w * (vc[j] - vu[j]);
        zn[j] = (j < 4 ? z0[j] : z1[j - 4]) + dt * g;
    }
    f32x4_t* zo = reinterpret_cast<f32x4_t*>(a.z_out + k * a.Cl + c8);
    zo[0] = f32x4_t{zn[0], zn[1], zn[2], zn[3]};
    zo[1] = f32x4_t{zn[4], zn[5], zn[6], zn[7]};
    if (a.x_next != nullptr) {
        const u32x4_t b = pack8(zn);
        st16(a.x_next + int64_t(r.x) * a.ld_x + c8, b);
        st16(a.x_next + int64_t(r.y) * a.ld_x + c8, b);
    }
}

}  // namespace

hipError_t launch_cfg_euler(const CfgEulerArgs& a, hipStream_t stream) {
    const int64_t threads = a.N * (a.Cl >> 3);
    if (threads == 0) return hipSuccess;
    hipLaunchKernelGGL(cfg_euler_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mf
