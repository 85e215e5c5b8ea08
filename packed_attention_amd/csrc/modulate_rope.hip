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
// registers (kept as packed bf16), reduced across the wavefront with DPP.  The kernel is HBM-bound: per
// token it reads and writes 2*C bf16 (plus the 16 bytes of pos/mod_row);
// the shift/scale rows are shared by all tokens of a sample and stay in L2.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kTokensPerBlock = 4;  // 4 wavefronts of 64 lanes

// Register pin between passes over the packed rows: the compiler must take
// the packed values as redefined here, so it widens them again in the next
// pass instead of keeping every widened fp32 copy live across passes.
template <int NCH>
__device__ __forceinline__ void keep_packed(u32x4_t (&pq)[NCH], u32x4_t (&pk)[NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(pq[i]), "+v"(pk[i]));
}

// Up to C = 3072: five wavefronts per SIMD (<= 96 VGPRs), so that all
// tokens of a 1024^2 pack (17 per CU) are resident at once.
template <int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH <= 6 ? 5 : 1))) void modulate_rope_kernel(
    ModRopeArgs a) {
    const int lane = threadIdx.x & 63;
    // wave-uniform (readfirstlane): the buffer resources below live in SGPRs
    const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    const int C = a.H * a.D;
    const int nch = C >> 3;

    // Both rows stay packed (bf16 pairs) in registers and are widened to
    // fp32 on the fly in each pass, which keeps the wavefront small enough
    // for five per SIMD.
    u32x4_t pq[NCH], pk[NCH];
    // Raw buffer resources over the two rows: chunks past the row (C not a
    // multiple of 512) read zeros and their stores are dropped, so no load or
    // store sits behind a branch and all of them are in flight at once.
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(a.q_in + t * a.ld_in, row_bytes);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(a.k_in + t * a.ld_in, row_bytes);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        pq[i] = bload16(q_rs, 16u * uint32_t(lane + kWave * i), 0);
        pk[i] = bload16(k_rs, 16u * uint32_t(lane + kWave * i), 0);
    }
    const bool mod = a.shift != nullptr;

    // Rotation angles of this lane's four pairs (the same in every head),
    // computed while the rows are in flight.  The angle pos * theta is formed
    // in fp64 and reduced to a fraction of a turn in [-1/2, 1/2]; the
    // hardware sine and cosine take turns, so the result carries only fp32
    // rounding for any position.
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

    float mq = 0.f, mk = 0.f, rq = 1.f, rk = 1.f;
    __amdgpu_buffer_rsrc_t sh_rs = make_rsrc(nullptr, 0), sc_rs = make_rsrc(nullptr, 0);
    if (mod) {
        // LayerNorm statistics (population variance) in fp32, two passes.
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                sq += bf_lo(pq[i][w]) + bf_hi(pq[i][w]);
                sk += bf_lo(pk[i][w]) + bf_hi(pk[i][w]);
            }
        const float invC = 1.0f / float(C);
        keep_packed(pq, pk);
        mq = wave_sum(sq) * invC;
        mk = wave_sum(sk) * invC;
        float vq = 0.f, vk = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const bool in = lane + kWave * i < nch;   // zero-filled chunks are not row data
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float q0 = bf_lo(pq[i][w]) - mq, q1 = bf_hi(pq[i][w]) - mq;
                const float k0 = bf_lo(pk[i][w]) - mk, k1 = bf_hi(pk[i][w]) - mk;
                vq += in ? q0 * q0 + q1 * q1 : 0.f;
                vk += in ? k0 * k0 + k1 * k1 : 0.f;
            }
        }
        keep_packed(pq, pk);
        rq = rsqrtf(wave_sum(vq) * invC + a.eps);
        rk = rsqrtf(wave_sum(vk) * invC + a.eps);
        const int64_t m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        sh_rs = make_rsrc(a.shift + m * C, row_bytes);
        sc_rs = make_rsrc(a.scale + m * C, row_bytes);
    }

    const __amdgpu_buffer_rsrc_t qo_rs = make_rsrc(a.q_out + t * a.ld_out, row_bytes);
    const __amdgpu_buffer_rsrc_t ko_rs = make_rsrc(a.k_out + t * a.ld_out, row_bytes);
    // The adaLN chunks are loaded one chunk ahead of the stores: a load
    // written after a store waits for it (the compiler cannot tell the
    // buffers apart), so each chunk would otherwise pay a full round trip.
    u32x4_t nsh = {0u, 0u, 0u, 0u}, nsc = {0u, 0u, 0u, 0u};
    if (mod) {
        nsh = bload16(sh_rs, 16u * uint32_t(lane), 0);
        nsc = bload16(sc_rs, 16u * uint32_t(lane), 0);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const uint32_t off = 16u * uint32_t(lane + kWave * i);
        float xq[8], xk[8];
        unpack8(pq[i], xq);
        unpack8(pk[i], xk);
        if (mod) {
            float fs[8], fc[8];
            unpack8(nsh, fs);
            unpack8(nsc, fc);
            if (i + 1 < NCH) {
                nsh = bload16(sh_rs, off + 16u * kWave, 0);
                nsc = bload16(sc_rs, off + 16u * kWave, 0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float g = 1.0f + fc[j];
                xq[j] = (xq[j] - mq) * rq * g + fs[j];
                xk[j] = (xk[j] - mk) * rk * g + fs[j];
            }
        }
        float oq[8], ok[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float c = cs[j], s = sn[j];
            oq[2 * j] = xq[2 * j] * c - xq[2 * j + 1] * s;
            oq[2 * j + 1] = xq[2 * j] * s + xq[2 * j + 1] * c;
            ok[2 * j] = xk[2 * j] * c - xk[2 * j + 1] * s;
            ok[2 * j + 1] = xk[2 * j] * s + xk[2 * j + 1] * c;
        }
        bstore16(qo_rs, off, 0, pack8(oq));
        bstore16(ko_rs, off, 0, pack8(ok));
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
