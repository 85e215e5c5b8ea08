// Fused adaLN modulation + multi-axis rotary embedding of q and k (gfx950).
//
// Fusion of adaptive normalisation and rotary embedding ahead of the
// attention: picx.dev summary of Mage-Flow, Methodology > Training
// Infrastructure; gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 3.
// Otimizacao de Nivel de Sistema > Kernels Fundidos.  Per-sample 2D rotary
// positions: gist.science, Metodologia > 2. NR-MMDiT; frame axis for editing:
// picx.dev, Methodology > Native-Resolution MMDiT.
//
// Layout and mapping.  One wavefront owns one token and processes its q row
// and its k row (C = H*D bf16 channels each).  Lane l holds the 16-byte
// chunks l, l+64, l+128, ... of a row, so every load and store is a fully
// coalesced 1 KiB wavefront access.  Because D divides 512, all chunks of a
// lane sit at the same in-head offset e0 = (8*l) mod D, so a lane needs only
// the four rotation angles of its pairs e0..e0+7 once per token, shared by q
// and k and by every head.  LayerNorm statistics are fp32, two-pass over
// registers, reduced across the wavefront.  The kernel is HBM-bound: per
// token it reads and writes 2*C bf16 (plus the 16 bytes of pos/mod_row);
// the shift/scale rows are shared by all tokens of a sample and stay in L2.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kTokensPerBlock = 4;  // 4 wavefronts of 64 lanes

template <int NCH>
__global__ __launch_bounds__(256) void modulate_rope_kernel(ModRopeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int C = a.H * a.D;
    const int nch = C >> 3;

    float xq[NCH][8], xk[NCH][8];
    const uint16_t* qrow = a.q_in + t * a.ld_in;
    const uint16_t* krow = a.k_in + t * a.ld_in;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = lane + kWave * i;
        u32x4_t vq = {0, 0, 0, 0}, vk = {0, 0, 0, 0};
        if (ci < nch) {
            vq = ld16(qrow + 8 * ci);
            vk = ld16(krow + 8 * ci);
        }
        unpack8(vq, xq[i]);
        unpack8(vk, xk[i]);
    }

    if (a.shift != nullptr) {
        // LayerNorm statistics (population variance) in fp32, two passes.
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sq += xq[i][j];
                sk += xk[i][j];
            }
        const float invC = 1.0f / float(C);
        const float mq = wave_sum(sq) * invC;
        const float mk = wave_sum(sk) * invC;
        float vq = 0.f, vk = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            if (lane + kWave * i < nch) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float dq = xq[i][j] - mq, dk = xk[i][j] - mk;
                    vq += dq * dq;
                    vk += dk * dk;
                }
            }
        }
        const float rq = rsqrtf(wave_sum(vq) * invC + a.eps);
        const float rk = rsqrtf(wave_sum(vk) * invC + a.eps);
        const int64_t m = a.mod_row[t];
        const uint16_t* sh = a.shift + m * C;
        const uint16_t* sc = a.scale + m * C;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ci = lane + kWave * i;
            if (ci < nch) {
                float fs[8], fc[8];
                unpack8(ld16(sh + 8 * ci), fs);
                unpack8(ld16(sc + 8 * ci), fc);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float g = 1.0f + fc[j];
                    xq[i][j] = (xq[i][j] - mq) * rq * g + fs[j];
                    xk[i][j] = (xk[i][j] - mk) * rk * g + fs[j];
                }
            }
        }
    }

    // Rotation angles of this lane's four pairs (same in every head).  The
    // angle pos * theta is formed in fp64 and reduced to [-pi, pi] before the
    // fp32 sincos, so its error stays at fp32 rounding level for any position.
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    const double p = double(a.pos[3 * t + axis]);
    float cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double phi = p * a.theta[e0 / 2 + j];
        const double turns = rint(phi * 0.15915494309189535);        // 1 / (2 pi)
        const float r = float(__builtin_fma(-turns, 6.283185307179586, phi));
        sincosf(r, &sn[j], &cs[j]);
    }

    uint16_t* qo = a.q_out + t * a.ld_out;
    uint16_t* ko = a.k_out + t * a.ld_out;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = lane + kWave * i;
        if (ci < nch) {
            float rq[8], rk[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float c = cs[j], s = sn[j];
                rq[2 * j] = xq[i][2 * j] * c - xq[i][2 * j + 1] * s;
                rq[2 * j + 1] = xq[i][2 * j] * s + xq[i][2 * j + 1] * c;
                rk[2 * j] = xk[i][2 * j] * c - xk[i][2 * j + 1] * s;
                rk[2 * j + 1] = xk[i][2 * j] * s + xk[i][2 * j + 1] * c;
            }
            st16(qo + 8 * ci, pack8(rq));
            st16(ko + 8 * ci, pack8(rk));
        }
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
            a.theta[pair++] = std::pow(double(a.rope_base), -2.0 * j / double(dims[ax]));
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
