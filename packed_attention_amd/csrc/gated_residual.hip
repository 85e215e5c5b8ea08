// Gated residual after the attention, optionally fused with the next
// sub-layer's adaLN modulation (gfx950).
//
// Gating and residual chains as fused kernels: picx.dev summary of
// Mage-Flow, Methodology > Training Infrastructure; gist.science "Resumo
// Tecnico: Mage-Flow", Metodologia > 3. Otimizacao de Nivel de Sistema >
// Kernels Fundidos (residual connections among the fused operator chains).
//
//   y = x + gate[m(t)] * o                       (fp32, rounded to bf16)
//   z = LN(y) * (1 + scale2[m(t)]) + shift2[m(t)] (LN of the fp32 y)
//
// One wavefront per token row of C channels; lane l owns the 16-byte chunks
// l, l+64, ... so each access is a coalesced 1 KiB wavefront transaction.
// HBM-bound: per token it reads x and o and writes y (and z).
#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kTokensPerBlock = 4;

// Up to C = 3072: five wavefronts per SIMD (<= 96 VGPRs), so that all
// tokens of a 1024^2 pack (17 per CU) are resident at once.
template <int NCH, bool kFusedNorm>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH <= 6 ? 5 : 1))) void
gated_residual_kernel(GatedResArgs a) {
    const int lane = threadIdx.x & 63;
    // wave-uniform (readfirstlane): the buffer resources below live in SGPRs
    const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    const int C = a.C;
    const int nch = C >> 3;
    const int64_t m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
    // Raw buffer resources over the rows: chunks past the row (C not a
    // multiple of 512) read zeros and their stores are dropped, so no load or
    // store sits behind a branch and all loads of the row are in flight at once.
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(a.x + t * C, row_bytes);
    const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(a.o + t * C, row_bytes);
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(a.gate + m * C, row_bytes);
    const __amdgpu_buffer_rsrc_t y_rs = make_rsrc(a.y + t * C, row_bytes);

    u32x4_t px[NCH], po[NCH], pg[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const uint32_t off = 16u * uint32_t(lane + kWave * i);
        px[i] = bload16(x_rs, off, 0);
        po[i] = bload16(o_rs, off, 0);
        pg[i] = bload16(g_rs, off, 0);
    }
    float y[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float fx[8], fo[8], fg[8];
        unpack8(px[i], fx);
        unpack8(po[i], fo);
        unpack8(pg[i], fg);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[i][j] = fx[j] + fg[j] * fo[j];
        bstore16(y_rs, 16u * uint32_t(lane + kWave * i), 0, pack8(y[i]));
    }
    if constexpr (kFusedNorm) {
        // LayerNorm of the fp32 y (population variance), two passes; the
        // zero-filled chunks past the row hold y = 0 and are left out of the
        // variance.
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) s += y[i][j];
        const float invC = 1.0f / float(C);
        const float mean = wave_sum(s) * invC;
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const bool in = lane + kWave * i < nch;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float d = y[i][j] - mean;
                v += in ? d * d : 0.f;
            }
        }
        const float rstd = rsqrtf(wave_sum(v) * invC + a.eps);
        const __amdgpu_buffer_rsrc_t sh_rs = make_rsrc(a.shift2 + m * C, row_bytes);
        const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(a.scale2 + m * C, row_bytes);
        const __amdgpu_buffer_rsrc_t z_rs = make_rsrc(a.z + t * C, row_bytes);
        // adaLN chunks loaded one chunk ahead of the stores (a load written
        // after a store would wait for it)
        u32x4_t nsh = bload16(sh_rs, 16u * uint32_t(lane), 0), nsc = bload16(sc_rs, 16u * uint32_t(lane), 0);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint32_t off = 16u * uint32_t(lane + kWave * i);
            float fs[8], fc[8], r[8];
            unpack8(nsh, fs);
            unpack8(nsc, fc);
            if (i + 1 < NCH) {
                nsh = bload16(sh_rs, off + 16u * kWave, 0);
                nsc = bload16(sc_rs, off + 16u * kWave, 0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) r[j] = (y[i][j] - mean) * rstd * (1.0f + fc[j]) + fs[j];
            bstore16(z_rs, off, 0, pack8(r));
        }
    }
}

template <int NCH>
hipError_t launch_nch(const GatedResArgs& a, hipStream_t stream) {
    const int64_t blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
    if (a.z != nullptr)
        hipLaunchKernelGGL((gated_residual_kernel<NCH, true>), dim3(unsigned(blocks)), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gated_residual_kernel<NCH, false>), dim3(unsigned(blocks)), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_residual(const GatedResArgs& a, hipStream_t stream) {
    const int nch = a.C / 8;
    const int per_lane = (nch + kWave - 1) / kWave;
    if (per_lane <= 1) return launch_nch<1>(a, stream);
    if (per_lane <= 2) return launch_nch<2>(a, stream);
    if (per_lane <= 4) return launch_nch<4>(a, stream);
    if (per_lane <= 6) return launch_nch<6>(a, stream);
    if (per_lane <= 8) return launch_nch<8>(a, stream);
    if (per_lane <= 12) return launch_nch<12>(a, stream);
    return launch_nch<16>(a, stream);
}

}  // namespace mf
