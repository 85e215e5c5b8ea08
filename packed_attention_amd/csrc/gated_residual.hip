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
// One workgroup per token row of C channels, each thread one 16-byte chunk
// (the workgroup is C/8 threads rounded up to whole wavefronts), so every
// access is a coalesced 1 KiB wavefront transaction and the grid streams
// reads and writes together (see the modulate + RoPE kernel for why this
// beats one wavefront per row).  The LayerNorm of the fused form reduces
// within wavefronts with DPP and across them through LDS.  HBM-bound: per
// token it reads x and o and writes y (and z); the gate and adaLN rows are
// shared by the tokens of a sample and stay in L2.
#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kMaxWaves = 16;       // C <= 8192: at most 1024 chunks per row

// Sum of v over the workgroup, in every thread (red: one float per wavefront
// of LDS, free again when this returns).
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < nw; ++i) s += red[i];
    __syncthreads();
    return s;
}

template <bool kFusedNorm>
__global__ __launch_bounds__(1024) void gated_residual_kernel(GatedResArgs a) {
    __shared__ float red[kMaxWaves];
    const int64_t t = blockIdx.x;
    const int c = threadIdx.x;                // this thread's chunk of the row
    const int C = a.C;
    const bool in = c < (C >> 3);
    // a row outside [0, n_rows) gets empty resources: its loads read zeros
    const int64_t m0 = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
    const bool mok = m0 >= 0 && m0 < a.n_rows;
    const int64_t m = mok ? m0 : 0;
    // Raw buffer resources over the rows: a chunk past the row reads zeros
    // and its store is dropped, so no load or store sits behind a branch.
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t mrow_bytes = mok ? row_bytes : 0u;
    const uint32_t off = 16u * uint32_t(c);
    const u32x4_t px = bload16(make_rsrc(a.x + t * C, row_bytes), off, 0);
    const u32x4_t po = bload16(make_rsrc(a.o + t * C, row_bytes), off, 0);
    const u32x4_t pg = bload16(make_rsrc(a.gate + m * C, mrow_bytes), off, 0);
    u32x4_t psh = {0u, 0u, 0u, 0u}, psc = {0u, 0u, 0u, 0u};
    if constexpr (kFusedNorm) {
        psh = bload16(make_rsrc(a.shift2 + m * C, mrow_bytes), off, 0);
        psc = bload16(make_rsrc(a.scale2 + m * C, mrow_bytes), off, 0);
    }
    float y[8];
    {
        float fx[8], fo[8], fg[8];
        unpack8(px, fx);
        unpack8(po, fo);
        unpack8(pg, fg);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = fx[j] + fg[j] * fo[j];
    }
    bstore16(make_rsrc(a.y + t * C, row_bytes), off, 0, pack8(y));
    if constexpr (kFusedNorm) {
        // LayerNorm of the fp32 y (population variance), two passes; chunks
        // past the row hold y = 0 and are left out of the variance.
        const float invC = 1.0f / float(C);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += y[j];
        const float mean = block_sum(s, red) * invC;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) v += (y[j] - mean) * (y[j] - mean);
        const float rstd = rsqrtf(block_sum(in ? v : 0.f, red) * invC + a.eps);
        float fs[8], fc[8], r[8];
        unpack8(psh, fs);
        unpack8(psc, fc);
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (y[j] - mean) * rstd * (1.0f + fc[j]) + fs[j];
        bstore16(make_rsrc(a.z + t * C, row_bytes), off, 0, pack8(r));
    }
}

}  // namespace

hipError_t launch_gated_residual(const GatedResArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int nch = a.C / 8;
    const int threads = (nch + kWave - 1) / kWave * kWave;   // <= 1024 for C <= 8192
    if (threads > kWave * kMaxWaves) return hipErrorInvalidConfiguration;
    if (a.z != nullptr)
        hipLaunchKernelGGL((gated_residual_kernel<true>), dim3(unsigned(a.T)), dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL((gated_residual_kernel<false>), dim3(unsigned(a.T)), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mf
