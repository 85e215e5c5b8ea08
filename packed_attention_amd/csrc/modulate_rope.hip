// Fused adaLN modulation + multi-axis rotary embedding of q and k (gfx950).
//
// Fusion of adaptive normalisation and rotary embedding ahead of the
// attention: picx.dev summary of Mage-Flow, Methodology > Training
// Infrastructure; gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 3.
// Otimizacao de Nivel de Sistema > Kernels Fundidos.  Per-sample 2D rotary
// positions: gist.science, Metodologia > 2. NR-MMDiT; frame axis for editing:
// picx.dev, Methodology > Native-Resolution MMDiT.
//
// Layout and mapping.  Two wavefronts per token: one takes the token's q row,
// the other its k row (C = H*D bf16 channels each).  Lane l holds the
// 16-byte chunks l, l+64, l+128, ... of the row, so every load and store is a
// fully coalesced 1 KiB wavefront access.  The sample's shift/scale rows
// (shared by all its tokens, so served from L2) are loaded together with the
// token's row, before the statistics, so no chunk waits for its adaLN values
// after the reductions.  Because D divides 512, all chunks of a lane sit at
// the same in-head offset e0 = (8*l) mod D, so a lane needs only the four
// rotation angles of its pairs e0..e0+7 once per token.  LayerNorm
// statistics are fp32, two-pass over registers (kept as packed bf16),
// reduced across the wavefront with DPP.  The kernel is HBM-bound: per token
// it reads and writes 2*C bf16 (plus the 16 bytes of pos/mod_row).
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kTokensPerBlock = 2;  // 4 wavefronts: q and k rows of two tokens

// Up to C = 3072: four wavefronts per SIMD (<= 128 VGPRs: the row and the two
// adaLN rows stay packed in registers).
template <int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH <= 6 ? 4 : 1))) void modulate_rope_kernel(
    ModRopeArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // two wavefronts per token: even ones take the q row, odd ones the k row
    const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (wave >> 1);
    const bool is_k = (wave & 1) != 0;
    if (t >= a.T) return;
    const int C = a.H * a.D;
    const int nch = C >> 3;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint16_t* in = is_k ? a.k_in : a.q_in;
    uint16_t* out = is_k ? a.k_out : a.q_out;
    const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(in + t * a.ld_in, row_bytes);
    u32x4_t px[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) px[i] = bload16(x_rs, 16u * uint32_t(lane + kWave * i), 0);
    const bool mod = a.shift != nullptr;
    u32x4_t ush[NCH], usc[NCH];
    if (mod) {
        // a row outside [0, n_rows) gets empty resources: its loads read zeros
        const int64_t m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        const bool mok = m >= 0 && m < a.n_rows;
        const __amdgpu_buffer_rsrc_t sh_rs = make_rsrc(a.shift + (mok ? m : 0) * C, mok ? row_bytes : 0u);
        const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(a.scale + (mok ? m : 0) * C, mok ? row_bytes : 0u);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            ush[i] = bload16(sh_rs, 16u * uint32_t(lane + kWave * i), 0);
            usc[i] = bload16(sc_rs, 16u * uint32_t(lane + kWave * i), 0);
        }
    }
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    const double p = double(a.pos[3 * t + axis]);
    float cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double turns = p * a.theta_turns[e0 / 2 + j];
        const float f = float(turns - rint(turns));
        sn[j] = __builtin_amdgcn_sinf(f);
        cs[j] = __builtin_amdgcn_cosf(f);
    }
    float mx = 0.f, rx = 1.f;
    if (mod) {
        float sx = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) sx += bf_lo(px[i][w]) + bf_hi(px[i][w]);
        const float invC = 1.0f / float(C);
        // Register pins between the passes: the compiler must take the packed
        // values as redefined here, so it widens them again in the next pass
        // instead of keeping every widened fp32 copy live.
#pragma unroll
        for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(px[i]));
        mx = wave_sum(sx) * invC;
        float vx = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const bool inr = lane + kWave * i < nch;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float x0 = bf_lo(px[i][w]) - mx, x1 = bf_hi(px[i][w]) - mx;
                vx += inr ? x0 * x0 + x1 * x1 : 0.f;
            }
        }
        rx = rsqrtf(wave_sum(vx) * invC + a.eps);
#pragma unroll
        for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(px[i]), "+v"(ush[i]), "+v"(usc[i]));
    }
    const __amdgpu_buffer_rsrc_t xo_rs = make_rsrc(out + t * a.ld_out, row_bytes);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const uint32_t off = 16u * uint32_t(lane + kWave * i);
        float x[8];
        unpack8(px[i], x);
        if (mod) {
            float fs[8], fc[8];
            unpack8(ush[i], fs);
            unpack8(usc[i], fc);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (x[j] - mx) * rx * (1.0f + fc[j]) + fs[j];
        }
        float o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = x[2 * j] * cs[j] - x[2 * j + 1] * sn[j];
            o[2 * j + 1] = x[2 * j] * sn[j] + x[2 * j + 1] * cs[j];
        }
        bstore16(xo_rs, off, 0, pack8(o));
    }
}

template <int NCH>
hipError_t launch_nch(const ModRopeArgs& a, hipStream_t stream) {
    const int64_t blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL(modulate_rope_kernel<NCH>, dim3(unsigned(blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_modulate_rope(const ModRopeArgs& args, hipStream_t stream) {
    ModRopeArgs a = args;
    // Frequency ladder of each axis block (frame, row, col), per pair of a head.
    const int dims[3] = {a.rope_f, a.rope_r, a.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            a.theta_turns[pair++] = std::pow(double(a.rope_base), -2.0 * j / double(dims[ax])) *
                                    0.15915494309189535;   // radians -> turns (1 / 2 pi)
    const int nch = (a.H * a.D) / 8;
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
