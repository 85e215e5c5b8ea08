// Backward of the fused elementwise kernels (gfx950): adaLN modulation +
// multi-axis RoPE of q and k, and the gated residual with the fused next
// adaLN.  The pages train the model with these fused kernels (picx.dev
// summary of Mage-Flow, Methodology > Training Infrastructure; gist.science
// "Resumo Tecnico: Mage-Flow", Metodologia > 3. Otimizacao de Nivel de
// Sistema > Kernels Fundidos); the gradients are the chain rule of the
// forward steps:
//   RoPE:      each pair's gradient turns back by -phi;
//   modulate:  u = xh (1 + scale) + shift, xh = (x - mu) / sigma:
//              gx = du (1 + scale), dx = (gx - mean gx - xh mean(gx xh)) / sigma,
//              dshift[r] += du, dscale[r] += du xh;
//   residual:  y = x + gate o, z = LN(y)(1 + scale2) + shift2:
//              dyt = dy + LN-backward(dz (1 + scale2)), dx = dyt,
//              do = gate dyt, dgate[r] += dyt o, dshift2[r] += dz,
//              dscale2[r] += dz yh.
//
// Layout and mapping.  One wavefront processes a run of kRun consecutive
// tokens; lane l holds the 16-byte chunks l, l+64, ... of every row, as in
// the forward kernels, so all global accesses are coalesced 1 KiB wavefront
// accesses.  Row statistics are fp32 wavefront reductions.  The per-row
// gradient sums (dshift, dscale, dgate, ...) are accumulated per lane in LDS
// while consecutive tokens share an adaLN row and flushed with fp32 global
// atomics when the row changes and at the end of the run, so a 1024^2 pack
// (one row per sample) issues about C atomics per run and sum instead of per
// token.  The order of those fp32 additions varies between runs (the row
// sums are not bitwise reproducible; everything else is).
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kRun = 4;   // tokens per wavefront

// Register pin between passes over packed rows: the compiler takes the
// packed values as redefined here, so it widens them again in the next pass
// instead of keeping every widened fp32 copy live across passes.
template <int N>
__device__ __forceinline__ void keep_packed(u32x4_t (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// fp32 global atomic add (global_atomic_add_f32), result unused.
__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t stream) {
    if (p == nullptr || n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

// Flush NA per-lane LDS partial arrays (each NCH chunks of 8 floats per lane)
// into rows `row` of NA global [n_rows][C] arrays, and clear them.
template <int NCH, int NA>
__device__ __forceinline__ void flush_rows(float* part, float* const (&dst)[NA], int row, int C, int lane) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c0 = 8 * (lane + kWave * i);
            if (c0 < C) {
                float* pp = part + (a * NCH + i) * 512 + 8 * lane;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    atomic_add_f32(dst[a] + int64_t(row) * C + c0 + j, pp[j]);
                    pp[j] = 0.f;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// modulate + RoPE backward
// ---------------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(64) void modulate_rope_bwd_kernel(ModRopeBwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) float part[];   // [2][NCH][64][8]
    const int lane = threadIdx.x;
    const int C = a.H * a.D;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const bool mod = a.scale != nullptr;
    const float invC = 1.0f / float(C);
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    if (mod)
        for (int i = 0; i < 2 * NCH * 8; ++i) part[(i / 8) * 512 + 8 * lane + (i % 8)] = 0.f;
    float* const dst[2] = {a.dshift, a.dscale};
    int cur = -1;
    for (int tt = 0; tt < kRun; ++tt) {
        const int64_t t = int64_t(blockIdx.x) * kRun + tt;
        if (t >= a.T) break;
        u32x4_t px[2][NCH], pg[2][NCH];          // q, k rows and their output gradients
        {
            const __amdgpu_buffer_rsrc_t rs[4] = {
                make_rsrc(a.q_in + t * a.ld_in, row_bytes), make_rsrc(a.k_in + t * a.ld_in, row_bytes),
                make_rsrc(a.dq_out + t * a.ld_gout, row_bytes), make_rsrc(a.dk_out + t * a.ld_gout, row_bytes)};
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const uint32_t off = 16u * uint32_t(lane + kWave * i);
                pg[0][i] = bload16(rs[2], off, 0);
                pg[1][i] = bload16(rs[3], off, 0);
                if (mod) {
                    px[0][i] = bload16(rs[0], off, 0);
                    px[1][i] = bload16(rs[1], off, 0);
                }
            }
        }
        // rotation angles of this lane's four pairs (as in the forward)
        const double p = double(a.pos[3 * t + axis]);
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = p * a.theta_turns[e0 / 2 + j];
            const float f = float(turns - rint(turns));
            sn[j] = __builtin_amdgcn_sinf(f);
            cs[j] = __builtin_amdgcn_cosf(f);
        }
        // gradient with respect to the RoPE input: each pair turned back
        auto rot_back = [&](const u32x4_t& v, float* g) {
            float h[8];
            unpack8(v, h);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                g[2 * j] = h[2 * j] * cs[j] + h[2 * j + 1] * sn[j];
                g[2 * j + 1] = -h[2 * j] * sn[j] + h[2 * j + 1] * cs[j];
            }
        };
        const __amdgpu_buffer_rsrc_t go[2] = {make_rsrc(a.dq_in + t * a.ld_gin, row_bytes),
                                              make_rsrc(a.dk_in + t * a.ld_gin, row_bytes)};
        if (!mod) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    float g[8];
                    rot_back(pg[x][i], g);
                    bstore16(go[x], 16u * uint32_t(lane + kWave * i), 0, pack8(g));
                }
            continue;
        }
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            if (cur >= 0) flush_rows<NCH, 2>(part, dst, cur, C, lane);
            cur = m;
        }
        const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(a.scale + int64_t(m) * C, row_bytes);
        keep_packed(px[0]); keep_packed(px[1]); keep_packed(pg[0]); keep_packed(pg[1]);
        // LayerNorm statistics of q and k rows (fp32, two passes)
        float mu[2], rs[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w) s += bf_lo(px[x][i][w]) + bf_hi(px[x][i][w]);
            mu[x] = wave_sum(s) * invC;
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const bool in = lane + kWave * i < (C >> 3);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float d0 = bf_lo(px[x][i][w]) - mu[x], d1 = bf_hi(px[x][i][w]) - mu[x];
                    v += in ? d0 * d0 + d1 * d1 : 0.f;
                }
            }
            rs[x] = rsqrtf(wave_sum(v) * invC + a.eps);
        }
        keep_packed(px[0]); keep_packed(px[1]); keep_packed(pg[0]); keep_packed(pg[1]);
        // pass 1: mean(gx), mean(gx xh) per row; row-sum partials
        float sa[2] = {0.f, 0.f}, sb[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint32_t off = 16u * uint32_t(lane + kWave * i);
            float sc[8];
            unpack8(bload16(sc_rs, off, 0), sc);
            float* psh = part + i * 512 + 8 * lane;
            float* psc = part + (NCH + i) * 512 + 8 * lane;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                float g[8], xv[8];
                rot_back(pg[x][i], g);
                unpack8(px[x][i], xv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float xh = (xv[j] - mu[x]) * rs[x];
                    const float gx = g[j] * (1.0f + sc[j]);
                    sa[x] += gx;
                    sb[x] += gx * xh;
                    psh[j] += g[j];
                    psc[j] += g[j] * xh;
                }
            }
        }
        float ma[2], mb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            ma[x] = wave_sum(sa[x]) * invC;
            mb[x] = wave_sum(sb[x]) * invC;
        }
        keep_packed(px[0]); keep_packed(px[1]); keep_packed(pg[0]); keep_packed(pg[1]);
        // pass 2: dx = (gx - mean gx - xh mean(gx xh)) / sigma
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint32_t off = 16u * uint32_t(lane + kWave * i);
            float sc[8];
            unpack8(bload16(sc_rs, off, 0), sc);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                float g[8], xv[8], dx[8];
                rot_back(pg[x][i], g);
                unpack8(px[x][i], xv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float xh = (xv[j] - mu[x]) * rs[x];
                    const float gx = g[j] * (1.0f + sc[j]);
                    dx[j] = (gx - ma[x] - xh * mb[x]) * rs[x];
                }
                bstore16(go[x], off, 0, pack8(dx));
            }
        }
    }
    if (mod && cur >= 0) flush_rows<NCH, 2>(part, dst, cur, C, lane);
}

// ---------------------------------------------------------------------------
// gated residual (+ fused next adaLN) backward
// ---------------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(64) void gated_residual_bwd_kernel(GatedResBwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) float part[];   // [3][NCH][64][8]
    const int lane = threadIdx.x;
    const int C = a.C;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const bool fused = a.dz != nullptr;
    const bool has_dy = a.dy != nullptr;
    const float invC = 1.0f / float(C);
    constexpr int NA = 3;
    for (int i = 0; i < NA * NCH * 8; ++i) part[(i / 8) * 512 + 8 * lane + (i % 8)] = 0.f;
    float* const dst[NA] = {a.dgate, a.dshift2, a.dscale2};
    int cur = -1;
    for (int tt = 0; tt < kRun; ++tt) {
        const int64_t t = int64_t(blockIdx.x) * kRun + tt;
        if (t >= a.T) break;
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            if (cur >= 0) {
                if (fused) flush_rows<NCH, 3>(part, dst, cur, C, lane);
                else flush_rows<NCH, 1>(part, reinterpret_cast<float* const(&)[1]>(dst), cur, C, lane);
            }
            cur = m;
        }
        const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(a.x + t * C, row_bytes);
        const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(a.o + t * C, row_bytes);
        const __amdgpu_buffer_rsrc_t g_rs = make_rsrc(a.gate + int64_t(m) * C, row_bytes);
        const __amdgpu_buffer_rsrc_t dy_rs = make_rsrc(has_dy ? a.dy + t * C : nullptr, has_dy ? row_bytes : 0);
        const __amdgpu_buffer_rsrc_t dz_rs = make_rsrc(fused ? a.dz + t * C : nullptr, fused ? row_bytes : 0);
        const __amdgpu_buffer_rsrc_t s2_rs = make_rsrc(fused ? a.scale2 + int64_t(m) * C : nullptr, fused ? row_bytes : 0);
        u32x4_t po[NCH], pdy[NCH], pdz[NCH];
        float y[NCH][8];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint32_t off = 16u * uint32_t(lane + kWave * i);
            const u32x4_t px = bload16(x_rs, off, 0);
            po[i] = bload16(o_rs, off, 0);
            pdy[i] = bload16(dy_rs, off, 0);     // zeros without dy
            pdz[i] = bload16(dz_rs, off, 0);     // zeros without dz
            float xv[8], ov[8], gv[8];
            unpack8(px, xv);
            unpack8(po[i], ov);
            unpack8(bload16(g_rs, off, 0), gv);
#pragma unroll
            for (int j = 0; j < 8; ++j) y[i][j] = xv[j] + gv[j] * ov[j];
        }
        keep_packed(po); keep_packed(pdy); keep_packed(pdz);
        float mu = 0.f, rs = 0.f, ma = 0.f, mb = 0.f;
        if (fused) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) s += y[i][j];        // zero-filled chunks give y = 0
            mu = wave_sum(s) * invC;
            float v = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const bool in = lane + kWave * i < (C >> 3);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float d = y[i][j] - mu;
                    v += in ? d * d : 0.f;
                }
            }
            rs = rsqrtf(wave_sum(v) * invC + a.eps);
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const uint32_t off = 16u * uint32_t(lane + kWave * i);
                float s2[8], dz[8];
                unpack8(bload16(s2_rs, off, 0), s2);
                unpack8(pdz[i], dz);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float yh = (y[i][j] - mu) * rs;
                    const float gy = dz[j] * (1.0f + s2[j]);
                    sa += gy;
                    sb += gy * yh;
                }
            }
            ma = wave_sum(sa) * invC;
            mb = wave_sum(sb) * invC;
        }
        keep_packed(po); keep_packed(pdy); keep_packed(pdz);
        const __amdgpu_buffer_rsrc_t dx_rs = make_rsrc(a.dx + t * C, row_bytes);
        const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(a.dout + t * C, row_bytes);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint32_t off = 16u * uint32_t(lane + kWave * i);
            float ov[8], gv[8], dy[8], dz[8], s2[8], dxo[8], doo[8];
            unpack8(po[i], ov);
            unpack8(bload16(g_rs, off, 0), gv);
            unpack8(pdy[i], dy);
            unpack8(pdz[i], dz);
            if (fused) unpack8(bload16(s2_rs, off, 0), s2);
            float* pgt = part + i * 512 + 8 * lane;
            float* psh = part + (NCH + i) * 512 + 8 * lane;
            float* psc = part + (2 * NCH + i) * 512 + 8 * lane;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float dyt = dy[j];
                if (fused) {
                    const float yh = (y[i][j] - mu) * rs;
                    const float gy = dz[j] * (1.0f + s2[j]);
                    dyt += (gy - ma - yh * mb) * rs;
                    psh[j] += dz[j];
                    psc[j] += dz[j] * yh;
                }
                dxo[j] = dyt;
                doo[j] = gv[j] * dyt;
                pgt[j] += dyt * ov[j];
            }
            bstore16(dx_rs, off, 0, pack8(dxo));
            bstore16(do_rs, off, 0, pack8(doo));
        }
    }
    if (cur >= 0) {
        if (fused) flush_rows<NCH, 3>(part, dst, cur, C, lane);
        else flush_rows<NCH, 1>(part, reinterpret_cast<float* const(&)[1]>(dst), cur, C, lane);
    }
}

template <int NCH>
hipError_t launch_modrope_bwd_nch(const ModRopeBwdArgs& a, hipStream_t stream) {
    const size_t lds = a.scale != nullptr ? size_t(2) * NCH * 512 * 4 : 0;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&modulate_rope_bwd_kernel<NCH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(size_t(2) * NCH * 512 * 4));
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (a.T + kRun - 1) / kRun;
    hipLaunchKernelGGL(modulate_rope_bwd_kernel<NCH>, dim3(unsigned(blocks)), dim3(64), lds, stream, a);
    return hipGetLastError();
}

template <int NCH>
hipError_t launch_gres_bwd_nch(const GatedResBwdArgs& a, hipStream_t stream) {
    const size_t lds = size_t(3) * NCH * 512 * 4;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gated_residual_bwd_kernel<NCH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (a.T + kRun - 1) / kRun;
    hipLaunchKernelGGL(gated_residual_bwd_kernel<NCH>, dim3(unsigned(blocks)), dim3(64), lds, stream, a);
    return hipGetLastError();
}

int chunks_per_lane(int C) { return (C / 8 + kWave - 1) / kWave; }

}  // namespace

hipError_t launch_modulate_rope_bwd(const ModRopeBwdArgs& args, hipStream_t stream) {
    ModRopeBwdArgs a = args;
    const int dims[3] = {a.rope_f, a.rope_r, a.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            a.theta_turns[pair++] = std::pow(double(a.rope_base), -2.0 * j / double(dims[ax])) *
                                    0.15915494309189535;   // radians -> turns (1 / 2 pi)
    const int64_t C = int64_t(a.H) * a.D;
    if (a.scale != nullptr) {
        hipError_t e = zero_f32(a.dshift, int64_t(a.n_rows) * C, stream);
        if (e == hipSuccess) e = zero_f32(a.dscale, int64_t(a.n_rows) * C, stream);
        if (e != hipSuccess) return e;
    }
    if (a.T == 0) return hipSuccess;
    const int per_lane = chunks_per_lane(int(C));
    if (per_lane <= 1) return launch_modrope_bwd_nch<1>(a, stream);
    if (per_lane <= 2) return launch_modrope_bwd_nch<2>(a, stream);
    if (per_lane <= 4) return launch_modrope_bwd_nch<4>(a, stream);
    if (per_lane <= 6) return launch_modrope_bwd_nch<6>(a, stream);
    if (per_lane <= 8) return launch_modrope_bwd_nch<8>(a, stream);
    if (per_lane <= 12) return launch_modrope_bwd_nch<12>(a, stream);
    return launch_modrope_bwd_nch<16>(a, stream);
}

hipError_t launch_gated_residual_bwd(const GatedResBwdArgs& a, hipStream_t stream) {
    const int64_t n = int64_t(a.n_rows) * a.C;
    hipError_t e = zero_f32(a.dgate, n, stream);
    if (e == hipSuccess && a.dz != nullptr) e = zero_f32(a.dshift2, n, stream);
    if (e == hipSuccess && a.dz != nullptr) e = zero_f32(a.dscale2, n, stream);
    if (e != hipSuccess) return e;
    if (a.T == 0) return hipSuccess;
    const int per_lane = chunks_per_lane(a.C);
    if (per_lane <= 1) return launch_gres_bwd_nch<1>(a, stream);
    if (per_lane <= 2) return launch_gres_bwd_nch<2>(a, stream);
    if (per_lane <= 4) return launch_gres_bwd_nch<4>(a, stream);
    if (per_lane <= 6) return launch_gres_bwd_nch<6>(a, stream);
    if (per_lane <= 8) return launch_gres_bwd_nch<8>(a, stream);
    if (per_lane <= 12) return launch_gres_bwd_nch<12>(a, stream);
    return launch_gres_bwd_nch<16>(a, stream);
}

}  // namespace mf
