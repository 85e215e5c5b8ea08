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
// Layout and mapping.  A workgroup processes a run of kRun consecutive
// tokens, one token row at a time; thread i owns the 16-byte chunk i of the
// row (8 channels), so every row access is one coalesced pass and each
// thread's per-row gradient sums are 8 registers per summed array.  Row
// statistics (LayerNorm mean and variance, then mean(gx) and mean(gx xh))
// are workgroup reductions: DPP within each wavefront, then the wavefront
// partials through LDS.  The next token's rows are loaded while the current
// one is reduced.
//
// Per-row sums over tokens (dshift, dscale, dgate, ...) without global
// contention: each workgroup keeps the sums of its current adaLN row in
// registers; a row change inside the run (a sample or modality boundary)
// adds the finished sums to the output with fp32 global atomics (rare), and
// at the end of the run the workgroup writes its sums once to its own slot
// of the caller's workspace, tagged with the row.  A second kernel then walks
// the slots in order, one thread per channel and group of slots, and adds
// each run of equal tags to the output row.  Each output row is touched by a
// handful of atomic adds instead of one per token, so a pack whose tokens all
// share one row (one sample) does not serialise on it.  The order of the fp32
// additions into the outputs varies between calls (the row sums are not
// bitwise reproducible; dx and the other per-token outputs are).
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kRun = 4;          // tokens per workgroup
constexpr int kSlotGroup = 32;   // slots summed per thread of the reduction kernel

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

// Workgroup sum of N values per thread; every thread receives the totals.
// `red` holds 2 * N * 16 floats; successive calls must alternate `buf`
// (0, 1, 0, ...) so that one barrier per call suffices.
template <int N>
__device__ __forceinline__ void wg_sum(float (&v)[N], float* red, int buf) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = (blockDim.x + 63) >> 6;
    float* r = red + buf * N * 16;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float s = wave_sum(v[k]);
        if (lane == 0) r[k * 16 + wave] = s;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += r[k * 16 + w];
        v[k] = s;
    }
}

// Slot layout of the workspace: tags [n_slots] (int32, 256-aligned block),
// then n_slots x NA x C floats.
__host__ __device__ constexpr size_t slot_tags_bytes(int64_t n_slots) {
    return (size_t(n_slots) * 4 + 255) / 256 * 256;
}
__host__ __device__ constexpr int64_t n_slots_for(int64_t T) { return (T + kRun - 1) / kRun; }

// Add the workspace slots to the outputs, one thread per (channel, group of
// kSlotGroup consecutive slots): runs of equal tags are summed in order and
// added to their row with one atomic add each.
template <int NA>
__global__ __launch_bounds__(256) void slot_reduce_kernel(const int32_t* __restrict__ tags,
                                                          const float* __restrict__ slots, int64_t n_slots,
                                                          int C, float* o0, float* o1, float* o2) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    float* const outs[3] = {o0, o1, o2};
    const int64_t s0 = int64_t(blockIdx.y) * kSlotGroup;
    const int64_t s1 = s0 + kSlotGroup < n_slots ? s0 + kSlotGroup : n_slots;
    int cur = -1;
    float acc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[a] = 0.f;
    for (int64_t s = s0; s < s1; ++s) {
        const int tag = tags[s];
        if (tag < 0) continue;
        if (tag != cur) {
            if (cur >= 0)
#pragma unroll
                for (int a = 0; a < NA; ++a) atomic_add_f32(outs[a] + int64_t(cur) * C + c, acc[a]);
            cur = tag;
#pragma unroll
            for (int a = 0; a < NA; ++a) acc[a] = 0.f;
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) acc[a] += slots[(s * NA + a) * C + c];
    }
    if (cur >= 0)
#pragma unroll
        for (int a = 0; a < NA; ++a) atomic_add_f32(outs[a] + int64_t(cur) * C + c, acc[a]);
}

// Finished row sums of this thread's 8 channels: to the output with
// atomics (row change inside a run) or to the workgroup's slot (end of run).
template <int NA>
__device__ __forceinline__ void rows_to_output(float (&p)[NA][8], float* const (&outs)[NA], int row, int C, int c0) {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            atomic_add_f32(outs[a] + int64_t(row) * C + c0 + j, p[a][j]);
            p[a][j] = 0.f;
        }
}
template <int NA>
__device__ __forceinline__ void rows_to_slot(const float (&p)[NA][8], float* slot, int C, int c0) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        f32x4_t lo = {p[a][0], p[a][1], p[a][2], p[a][3]};
        f32x4_t hi = {p[a][4], p[a][5], p[a][6], p[a][7]};
        *reinterpret_cast<f32x4_t*>(slot + int64_t(a) * C + c0) = lo;
        *reinterpret_cast<f32x4_t*>(slot + int64_t(a) * C + c0 + 4) = hi;
    }
}

// ---------------------------------------------------------------------------
// modulate + RoPE backward
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void modulate_rope_bwd_kernel(ModRopeBwdArgs a) {
    __shared__ float red[2 * 4 * 16];
    const int C = a.H * a.D;
    const int ci = threadIdx.x;                 // this thread's chunk
    const bool live = ci < (C >> 3);
    const int c0 = 8 * ci;
    const bool mod = a.scale != nullptr;
    const float invC = 1.0f / float(C);
    const int e0 = c0 % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    double th[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) th[j] = a.theta_turns[e0 / 2 + j];
    const int64_t t_begin = int64_t(blockIdx.x) * kRun;
    const int64_t t_end = t_begin + kRun < a.T ? t_begin + kRun : a.T;
    float* const outs[2] = {a.dshift, a.dscale};
    float part[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[0][j] = part[1][j] = 0.f;
    int cur = -1;
    int buf = 0;

    // rows of token t: output gradients of q and k, then q and k
    auto load = [&](int64_t t, u32x4_t (&r)[4]) {
        if (live) {
            r[0] = ld16(a.dq_out + t * a.ld_gout + c0);
            r[1] = ld16(a.dk_out + t * a.ld_gout + c0);
            if (mod) {
                r[2] = ld16(a.q_in + t * a.ld_in + c0);
                r[3] = ld16(a.k_in + t * a.ld_in + c0);
            }
        }
    };
    u32x4_t nxt[4] = {};
    load(t_begin, nxt);
    for (int64_t t = t_begin; t < t_end; ++t) {
        u32x4_t row[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) row[i] = nxt[i];
        if (t + 1 < t_end) load(t + 1, nxt);

        // gradient with respect to the RoPE input: each pair turned back
        float g[2][8];
        {
            const double p = double(a.pos[3 * t + axis]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double turns = p * th[j];
                const float f = float(turns - rint(turns));
                const float s = __builtin_amdgcn_sinf(f), c = __builtin_amdgcn_cosf(f);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const float h0 = bf_lo(row[x][j]), h1 = bf_hi(row[x][j]);
                    g[x][2 * j] = h0 * c + h1 * s;
                    g[x][2 * j + 1] = -h0 * s + h1 * c;
                }
            }
        }
        uint16_t* const dst[2] = {a.dq_in + t * a.ld_gin + c0, a.dk_in + t * a.ld_gin + c0};
        if (!mod) {
            if (live) {
                st16(dst[0], pack8(g[0]));
                st16(dst[1], pack8(g[1]));
            }
            continue;
        }
        const int m = a.mod_row[t];
        if (m != cur) {
            if (cur >= 0 && live) rows_to_output<2>(part, outs, cur, C, c0);
            cur = m;
        }
        float x[2][8];
        unpack8(row[2], x[0]);
        unpack8(row[3], x[1]);
        // LayerNorm statistics of the q and k rows (fp32, two passes)
        float st[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            st[0] += x[0][j];
            st[1] += x[1][j];
        }
        wg_sum<4>(st, red, buf);
        buf ^= 1;
        const float mu[2] = {st[0] * invC, st[1] * invC};
        float vr[4] = {0.f, 0.f, 0.f, 0.f};
        if (live)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                vr[0] += (x[0][j] - mu[0]) * (x[0][j] - mu[0]);
                vr[1] += (x[1][j] - mu[1]) * (x[1][j] - mu[1]);
            }
        wg_sum<4>(vr, red, buf);
        buf ^= 1;
        const float rs[2] = {rsqrtf(vr[0] * invC + a.eps), rsqrtf(vr[1] * invC + a.eps)};
        float sc[8];
        unpack8(live ? ld16(a.scale + int64_t(m) * C + c0) : u32x4_t{}, sc);
        float xh[2][8], gx[2][8];
        float ab[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                xh[q][j] = (x[q][j] - mu[q]) * rs[q];
                gx[q][j] = g[q][j] * (1.0f + sc[j]);
                ab[2 * q] += gx[q][j];
                ab[2 * q + 1] += gx[q][j] * xh[q][j];
            }
        wg_sum<4>(ab, red, buf);
        buf ^= 1;
        if (live) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float dx[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    dx[j] = (gx[q][j] - ab[2 * q] * invC - xh[q][j] * ab[2 * q + 1] * invC) * rs[q];
                st16(dst[q], pack8(dx));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                part[0][j] += g[0][j] + g[1][j];
                part[1][j] += g[0][j] * xh[0][j] + g[1][j] * xh[1][j];
            }
        }
    }
    if (mod) {
        int32_t* tags = static_cast<int32_t*>(a.workspace);
        float* slot = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) +
                                               slot_tags_bytes(n_slots_for(a.T))) +
                      int64_t(blockIdx.x) * 2 * C;
        if (live) rows_to_slot<2>(part, slot, C, c0);
        if (threadIdx.x == 0) tags[blockIdx.x] = cur;
    }
}

// ---------------------------------------------------------------------------
// gated residual (+ fused next adaLN) backward
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gated_residual_bwd_kernel(GatedResBwdArgs a) {
    __shared__ float red[2 * 2 * 16];
    const int C = a.C;
    const int ci = threadIdx.x;
    const bool live = ci < (C >> 3);
    const int c0 = 8 * ci;
    const bool fused = a.dz != nullptr;
    const bool has_dy = a.dy != nullptr;
    const float invC = 1.0f / float(C);
    const int64_t t_begin = int64_t(blockIdx.x) * kRun;
    const int64_t t_end = t_begin + kRun < a.T ? t_begin + kRun : a.T;
    float* const outs[3] = {a.dgate, a.dshift2, a.dscale2};
    float part[3][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[0][j] = part[1][j] = part[2][j] = 0.f;
    int cur = -1;
    int buf = 0;

    // rows of token t: x, o, dy, dz
    auto load = [&](int64_t t, u32x4_t (&r)[4]) {
        if (live) {
            r[0] = ld16(a.x + t * C + c0);
            r[1] = ld16(a.o + t * C + c0);
            if (has_dy) r[2] = ld16(a.dy + t * C + c0);
            if (fused) r[3] = ld16(a.dz + t * C + c0);
        }
    };
    u32x4_t nxt[4] = {};
    load(t_begin, nxt);
    for (int64_t t = t_begin; t < t_end; ++t) {
        u32x4_t row[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) row[i] = nxt[i];
        if (t + 1 < t_end) load(t + 1, nxt);
        const int m = a.mod_row[t];
        if (m != cur) {
            if (cur >= 0 && live) {
                if (fused)
                    rows_to_output<3>(part, outs, cur, C, c0);
                else
                    rows_to_output<1>(reinterpret_cast<float(&)[1][8]>(part),
                                      reinterpret_cast<float* const(&)[1]>(outs), cur, C, c0);
            }
            cur = m;
        }
        float xv[8], ov[8], gv[8], dy[8], dz[8];
        unpack8(row[0], xv);
        unpack8(row[1], ov);
        unpack8(live ? ld16(a.gate + int64_t(m) * C + c0) : u32x4_t{}, gv);
        unpack8(has_dy ? row[2] : u32x4_t{}, dy);
        unpack8(fused ? row[3] : u32x4_t{}, dz);
        float y[8], dyt[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = xv[j] + gv[j] * ov[j];
            dyt[j] = dy[j];
        }
        if (fused) {
            float s[2] = {0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) s[0] += y[j];          // dead chunks hold y = 0
            wg_sum<2>(s, red, buf);
            buf ^= 1;
            const float mu = s[0] * invC;
            float v[2] = {0.f, 0.f};
            if (live)
#pragma unroll
                for (int j = 0; j < 8; ++j) v[0] += (y[j] - mu) * (y[j] - mu);
            wg_sum<2>(v, red, buf);
            buf ^= 1;
            const float rs = rsqrtf(v[0] * invC + a.eps);
            float s2[8];
            unpack8(live ? ld16(a.scale2 + int64_t(m) * C + c0) : u32x4_t{}, s2);
            float yh[8], gy[8];
            float ab[2] = {0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                yh[j] = (y[j] - mu) * rs;
                gy[j] = dz[j] * (1.0f + s2[j]);
                ab[0] += gy[j];
                ab[1] += gy[j] * yh[j];
            }
            wg_sum<2>(ab, red, buf);
            buf ^= 1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                dyt[j] += (gy[j] - ab[0] * invC - yh[j] * ab[1] * invC) * rs;
                part[1][j] += dz[j];
                part[2][j] += dz[j] * yh[j];
            }
        }
        if (live) {
            float dov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                dov[j] = gv[j] * dyt[j];
                part[0][j] += dyt[j] * ov[j];
            }
            st16(a.dx + t * C + c0, pack8(dyt));
            st16(a.dout + t * C + c0, pack8(dov));
        }
    }
    const int na = fused ? 3 : 1;
    int32_t* tags = static_cast<int32_t*>(a.workspace);
    float* slot = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) +
                                           slot_tags_bytes(n_slots_for(a.T))) +
                  int64_t(blockIdx.x) * na * C;
    if (live) {
        if (fused)
            rows_to_slot<3>(part, slot, C, c0);
        else
            rows_to_slot<1>(reinterpret_cast<float(&)[1][8]>(part), slot, C, c0);
    }
    if (threadIdx.x == 0) tags[blockIdx.x] = cur;
}

int block_threads(int C) { return ((C / 8 + 63) / 64) * 64; }

template <int NA>
hipError_t reduce_slots(void* ws, int64_t T, int C, float* o0, float* o1, float* o2, hipStream_t stream) {
    const int64_t ns = n_slots_for(T);
    const int32_t* tags = static_cast<const int32_t*>(ws);
    const float* slots = reinterpret_cast<const float*>(static_cast<const unsigned char*>(ws) + slot_tags_bytes(ns));
    dim3 grid(unsigned((C + 255) / 256), unsigned((ns + kSlotGroup - 1) / kSlotGroup));
    hipLaunchKernelGGL(slot_reduce_kernel<NA>, grid, dim3(256), 0, stream, tags, slots, ns, C, o0, o1, o2);
    return hipGetLastError();
}

}  // namespace

size_t elementwise_bwd_workspace_bytes(int64_t T, int32_t C, int32_t n_arrays) {
    const int64_t ns = n_slots_for(T < 0 ? 0 : T);
    return slot_tags_bytes(ns) + size_t(ns) * size_t(n_arrays) * size_t(C) * 4;
}

hipError_t launch_modulate_rope_bwd(const ModRopeBwdArgs& args, hipStream_t stream) {
    ModRopeBwdArgs a = args;
    const int dims[3] = {a.rope_f, a.rope_r, a.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            a.theta_turns[pair++] = std::pow(double(a.rope_base), -2.0 * j / double(dims[ax])) *
                                    0.15915494309189535;   // radians -> turns (1 / 2 pi)
    const int C = a.H * a.D;
    const bool mod = a.scale != nullptr;
    if (mod) {
        hipError_t e = zero_f32(a.dshift, int64_t(a.n_rows) * C, stream);
        if (e == hipSuccess) e = zero_f32(a.dscale, int64_t(a.n_rows) * C, stream);
        if (e != hipSuccess) return e;
    }
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(modulate_rope_bwd_kernel, dim3(unsigned(n_slots_for(a.T))), dim3(block_threads(C)), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !mod) return e;
    return reduce_slots<2>(a.workspace, a.T, C, a.dshift, a.dscale, nullptr, stream);
}

hipError_t launch_gated_residual_bwd(const GatedResBwdArgs& a, hipStream_t stream) {
    const int64_t n = int64_t(a.n_rows) * a.C;
    const bool fused = a.dz != nullptr;
    hipError_t e = zero_f32(a.dgate, n, stream);
    if (e == hipSuccess && fused) e = zero_f32(a.dshift2, n, stream);
    if (e == hipSuccess && fused) e = zero_f32(a.dscale2, n, stream);
    if (e != hipSuccess) return e;
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(gated_residual_bwd_kernel, dim3(unsigned(n_slots_for(a.T))), dim3(block_threads(a.C)),
                       0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (fused) return reduce_slots<3>(a.workspace, a.T, a.C, a.dgate, a.dshift2, a.dscale2, stream);
    return reduce_slots<1>(a.workspace, a.T, a.C, a.dgate, nullptr, nullptr, stream);
}

}  // namespace mf
