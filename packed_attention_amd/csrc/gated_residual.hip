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

template <int NCH, bool kFusedNorm>
__global__ __launch_bounds__(256) void gated_residual_kernel(GatedResArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int C = a.C;
    const int nch = C >> 3;
    const int64_t m = a.mod_row[t];
    const uint16_t* xr = a.x + t * C;
    const uint16_t* orow = a.o + t * C;
    const uint16_t* gr = a.gate + m * C;
    uint16_t* yr = a.y + t * C;

    float y[NCH][8];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = lane + kWave * i;
        if (ci < nch) {
            float fx[8], fo[8], fg[8];
            unpack8(ld16(xr + 8 * ci), fx);
            unpack8(ld16(orow + 8 * ci), fo);
            unpack8(ld16(gr + 8 * ci), fg);
#pragma unroll
            for (int j = 0; j < 8; ++j) y[i][j] = fx[j] + fg[j] * fo[j];
            st16(yr + 8 * ci, pack8(y[i]));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) y[i][j] = 0.f;
        }
    }
    if constexpr (kFusedNorm) {
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
            if (lane + kWave * i < nch) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float d = y[i][j] - mean;
                    v += d * d;
                }
            }
        }
        const float rstd = rsqrtf(wave_sum(v) * invC + a.eps);
        const uint16_t* sh = a.shift2 + m * C;
        const uint16_t* sc = a.scale2 + m * C;
        uint16_t* zr = a.z + t * C;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ci = lane + kWave * i;
            if (ci < nch) {
                float fs[8], fc[8], r[8];
                unpack8(ld16(sh + 8 * ci), fs);
                unpack8(ld16(sc + 8 * ci), fc);
#pragma unroll
                for (int j = 0; j < 8; ++j) r[j] = (y[i][j] - mean) * rstd * (1.0f + fc[j]) + fs[j];
                st16(zr + 8 * ci, pack8(r));
            }
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
