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
// Layout and mapping.  Each call runs two kernels and a reduction:
//  * the per-token outputs (dq, dk; dx, do) with the forward kernels'
//    mappings (modulate + RoPE: one wavefront per q or k row, statistics
//    inside the wavefront; gated residual: one workgroup per token, one
//    16-byte chunk per thread, LayerNorm reductions through LDS), which also
//    write each row's fp32 statistics (4 floats per token);
//  * the per-row sums over tokens (dshift, dscale; dgate, dshift2,
//    dscale2): one lane per 8-channel chunk walks a run of kSumRun tokens,
//    reads the rows again and recomputes the fp32 gradients from them and
//    the statistics, so the sums see the same fp32 values as the outputs;
//  * slot_reduce_kernel: each run leaves its sums in its own slot of the
//    caller's workspace, tagged with its adaLN row, and the reduction walks
//    the slots in order, one thread per channel and group of slots, adding
//    each run of equal tags to the output row with one fp32 atomic add.  A
//    row change inside a run adds the finished sums with atomics too.  Each
//    output row is touched by a handful of atomic adds instead of one per
//    token, so a pack whose tokens all share one row does not serialise on
//    it; the order of those additions varies between calls (the row sums
//    are not bitwise reproducible; every per-token output is).
// Modulate + RoPE rows of more than 3072 channels keep a single kernel: a
// workgroup walks a run of kRun tokens one row at a time (thread per chunk,
// statistics by workgroup reductions), keeps the sums of its current adaLN
// row in registers and writes them to its slot at the end of the run.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kRun = 4;          // tokens per workgroup
constexpr int kSlotGroup = 8;    // slots summed per thread of the reduction kernel

__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

// Zeros n floats at each of up to three arrays (blockIdx.y picks the array;
// nullptr entries are skipped), one launch for all of a call's row sums.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p0, float* __restrict__ p1,
                                                        float* __restrict__ p2, int64_t n) {
    float* const p = blockIdx.y == 0 ? p0 : blockIdx.y == 1 ? p1 : p2;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (p != nullptr && i < n) p[i] = 0.f;
}

hipError_t zero_f32(float* p0, float* p1, float* p2, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256), 3), dim3(256), 0, stream, p0, p1, p2, n);
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
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= C) return;
    float* const outs[3] = {o0, o1, o2};
    const int64_t s0 = int64_t(blockIdx.x) * kSlotGroup;
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
        const bool mok = m >= 0 && m < a.n_rows;      // a row outside the table reads zeros, adds nothing
        if (m != cur) {
            if (cur >= 0 && cur < a.n_rows && live) rows_to_output<2>(part, outs, cur, C, c0);
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
        unpack8(live && mok ? ld16(a.scale + int64_t(m) * C + c0) : u32x4_t{}, sc);
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
        if (threadIdx.x == 0) tags[blockIdx.x] = cur < a.n_rows ? cur : -1;   // -1: nothing to add
    }
}

// ---------------------------------------------------------------------------
// modulate + RoPE backward in two kernels (C <= 3072)
// ---------------------------------------------------------------------------
// Kernel A, the per-token outputs, with the forward kernel's mapping: one
// wavefront per row (q or k) of a token, two tokens per workgroup; lane l
// owns the 16-byte chunks l, l+64, ... (all at in-head offset 8l mod D, so
// its four rotation angles serve every chunk); the row statistics are
// reductions inside the wavefront.  It writes dq, dk and each row's mean and
// 1/sigma (fp32).  Kernel B, the per-row sums: lane = one 8-channel chunk of
// a run of kSumRun tokens; it reads the rows again, turns dq', dk' back and
// normalises q, k with kernel A's statistics, and writes one tagged slot
// per run (a row change inside a run adds the finished sums with atomics, as
// above); slot_reduce_kernel then adds the slots.  Reading the four rows
// twice costs less than keeping 2 x 8 fp32 sums per chunk in every
// wavefront, which does not fit two wavefronts per SIMD at C = 3072.
constexpr int kRowsTokens = 2;    // tokens per kernel-A workgroup
constexpr int kSumRun = 8;        // tokens per kernel-B slot
__host__ __device__ constexpr int64_t sum_slots_for(int64_t T) { return (T + kSumRun - 1) / kSumRun; }

template <int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH >= 6 ? 3 : 4))) void modrope_bwd_dx_kernel(
    ModRopeBwdArgs a, float* __restrict__ stats) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = int64_t(blockIdx.x) * kRowsTokens + (wave >> 1);
    const bool is_k = (wave & 1) != 0;
    if (t >= a.T) return;
    const int C = a.H * a.D;
    const int nch = C >> 3;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const bool mod = a.scale != nullptr;
    auto off = [&](int i) { return 16u * uint32_t(lane + kWave * i); };
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc((is_k ? a.dk_out : a.dq_out) + t * a.ld_gout, row_bytes);
    u32x4_t pg[NCH], px[NCH], usc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) pg[i] = bload16(g_rs, off(i), 0);
    if (mod) {
        const __amdgpu_buffer_rsrc_t x_rs = make_rsrc((is_k ? a.k_in : a.q_in) + t * a.ld_in, row_bytes);
        // a row outside [0, n_rows) reads zeros
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        const bool mok = m >= 0 && m < a.n_rows;
        const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(a.scale + int64_t(mok ? m : 0) * C, mok ? row_bytes : 0u);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            px[i] = bload16(x_rs, off(i), 0);
            usc[i] = bload16(sc_rs, off(i), 0);
        }
    }
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    float cs[4], sn[4];
    {
        const double p = double(a.pos[3 * t + axis]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = p * a.theta_turns[e0 / 2 + j];
            const float f = float(turns - rint(turns));
            sn[j] = __builtin_amdgcn_sinf(f);
            cs[j] = __builtin_amdgcn_cosf(f);
        }
    }
    // gradient with respect to the RoPE input: each pair turned back
    auto rot_back = [&](int i, float (&g)[8]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float h0 = bf_lo(pg[i][j]), h1 = bf_hi(pg[i][j]);
            g[2 * j] = h0 * cs[j] + h1 * sn[j];
            g[2 * j + 1] = -h0 * sn[j] + h1 * cs[j];
        }
    };
    const __amdgpu_buffer_rsrc_t d_rs = make_rsrc((is_k ? a.dk_in : a.dq_in) + t * a.ld_gin, row_bytes);
    if (!mod) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            float g[8];
            rot_back(i, g);
            bstore16(d_rs, off(i), 0, pack8(g));
        }
        return;
    }
    const float invC = 1.0f / float(C);
    // Register pins between the passes: the packed rows count as redefined
    // at each pin, so every pass widens them again instead of keeping the
    // widened fp32 copies live across the reductions.
    auto pin = [&] {
#pragma unroll
        for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(px[i]), "+v"(pg[i]), "+v"(usc[i]));
    };
    float sx = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) sx += bf_lo(px[i][w]) + bf_hi(px[i][w]);
    pin();
    const float mu = wave_sum(sx) * invC;
    float vx = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const bool inr = lane + kWave * i < nch;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float x0 = bf_lo(px[i][w]) - mu, x1 = bf_hi(px[i][w]) - mu;
            vx += inr ? x0 * x0 + x1 * x1 : 0.f;
        }
    }
    pin();
    const float rs = rsqrtf(wave_sum(vx) * invC + a.eps);
    // mean(gx) and mean(gx xh), gx = g (1 + scale); chunks past the row have g = 0
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float g[8], x[8], sc[8];
        rot_back(i, g);
        unpack8(px[i], x);
        unpack8(usc[i], sc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float gx = g[j] * (1.0f + sc[j]);
            sa += gx;
            sb += gx * ((x[j] - mu) * rs);
        }
    }
    pin();
    const float ma = wave_sum(sa) * invC, mb = wave_sum(sb) * invC;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float g[8], x[8], sc[8], dx[8];
        rot_back(i, g);
        unpack8(px[i], x);
        unpack8(usc[i], sc);
#pragma unroll
        for (int j = 0; j < 8; ++j) dx[j] = (g[j] * (1.0f + sc[j]) - ma - (x[j] - mu) * rs * mb) * rs;
        bstore16(d_rs, off(i), 0, pack8(dx));
    }
    if (lane == 0) *reinterpret_cast<float2*>(stats + 4 * t + 2 * (is_k ? 1 : 0)) = float2{mu, rs};
}

// Kernel B: blockIdx.x = run of kSumRun tokens, blockIdx.y = group of 64
// chunks; lane = one chunk (in-head offset 8l mod D, as in kernel A).
__global__ __launch_bounds__(64) void modrope_bwd_sums_kernel(ModRopeBwdArgs a, const float* __restrict__ stats,
                                                              int32_t* __restrict__ tags, float* __restrict__ slots) {
    const int lane = threadIdx.x;
    const int C = a.H * a.D;
    const int nch = C >> 3;
    const int c = blockIdx.y * kWave + lane;
    const bool live = c < nch;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t voff = 16u * uint32_t(c);
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    double th[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) th[j] = a.theta_turns[e0 / 2 + j];
    const int64_t t_begin = int64_t(blockIdx.x) * kSumRun;
    const int64_t t_end = t_begin + kSumRun < a.T ? t_begin + kSumRun : a.T;
    float s0[8], s1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s0[j] = s1[j] = 0.f;
    int cur = -1;
    auto flush = [&](int row) {
        if (row < 0 || row >= a.n_rows || !live) return;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            atomic_add_f32(a.dshift + int64_t(row) * C + 8 * c + j, s0[j]);
            atomic_add_f32(a.dscale + int64_t(row) * C + 8 * c + j, s1[j]);
            s0[j] = s1[j] = 0.f;
        }
    };
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            flush(cur);
            cur = m;
        }
        const u32x4_t gq = bload16(make_rsrc(a.dq_out + t * a.ld_gout, row_bytes), voff, 0);
        const u32x4_t gk = bload16(make_rsrc(a.dk_out + t * a.ld_gout, row_bytes), voff, 0);
        const u32x4_t xq = bload16(make_rsrc(a.q_in + t * a.ld_in, row_bytes), voff, 0);
        const u32x4_t xk = bload16(make_rsrc(a.k_in + t * a.ld_in, row_bytes), voff, 0);
        const f32x4_t st = *reinterpret_cast<const f32x4_t*>(stats + 4 * t);   // mu_q, rs_q, mu_k, rs_k
        const double p = double(a.pos[3 * t + axis]);
        if (m < 0 || m >= a.n_rows) continue;   // a row outside the table adds nothing
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = p * th[j];
            const float f = float(turns - rint(turns));
            const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
            const float q0 = bf_lo(gq[j]), q1 = bf_hi(gq[j]), k0 = bf_lo(gk[j]), k1 = bf_hi(gk[j]);
            const float gq0 = q0 * cs + q1 * sn, gq1 = -q0 * sn + q1 * cs;
            const float gk0 = k0 * cs + k1 * sn, gk1 = -k0 * sn + k1 * cs;
            const float hq0 = (bf_lo(xq[j]) - st[0]) * st[1], hq1 = (bf_hi(xq[j]) - st[0]) * st[1];
            const float hk0 = (bf_lo(xk[j]) - st[2]) * st[3], hk1 = (bf_hi(xk[j]) - st[2]) * st[3];
            s0[2 * j] += gq0 + gk0;
            s0[2 * j + 1] += gq1 + gk1;
            s1[2 * j] += gq0 * hq0 + gk0 * hk0;
            s1[2 * j + 1] += gq1 * hq1 + gk1 * hk1;
        }
    }
    float* slot = slots + int64_t(blockIdx.x) * 2 * C;
    if (live) {
        *reinterpret_cast<f32x4_t*>(slot + 8 * c) = f32x4_t{s0[0], s0[1], s0[2], s0[3]};
        *reinterpret_cast<f32x4_t*>(slot + 8 * c + 4) = f32x4_t{s0[4], s0[5], s0[6], s0[7]};
        *reinterpret_cast<f32x4_t*>(slot + C + 8 * c) = f32x4_t{s1[0], s1[1], s1[2], s1[3]};
        *reinterpret_cast<f32x4_t*>(slot + C + 8 * c + 4) = f32x4_t{s1[4], s1[5], s1[6], s1[7]};
    }
    if (blockIdx.y == 0 && lane == 0) tags[blockIdx.x] = cur >= 0 && cur < a.n_rows ? cur : -1;
}

int block_threads(int C) { return ((C / 8 + 63) / 64) * 64; }

template <int NA>
hipError_t reduce_slots(void* ws, int64_t T, int C, float* o0, float* o1, float* o2, hipStream_t stream) {
    const int64_t ns = n_slots_for(T);
    const int32_t* tags = static_cast<const int32_t*>(ws);
    const float* slots = reinterpret_cast<const float*>(static_cast<const unsigned char*>(ws) + slot_tags_bytes(ns));
    dim3 grid(unsigned((ns + kSlotGroup - 1) / kSlotGroup), unsigned((C + 255) / 256));
    hipLaunchKernelGGL(slot_reduce_kernel<NA>, grid, dim3(256), 0, stream, tags, slots, ns, C, o0, o1, o2);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gated residual backward in two kernels
// ---------------------------------------------------------------------------
// Kernel A: one workgroup per token, one 16-byte chunk per thread (the
// forward kernel's mapping), LayerNorm reductions through LDS; it writes dx,
// do and, with the fused adaLN, the token's mean and 1/sigma of y and the
// means of g2 and g2 yh (g2 = dz (1 + scale2)).  Kernel B: lane = one
// 8-channel chunk of a run of kSumRun tokens; it recomputes dyt in fp32 from
// the rows and those statistics and writes one tagged slot of dgate (and
// dshift2, dscale2) per run, as the modulate + RoPE sums kernel does.
template <bool FUSED>
__global__ __launch_bounds__(1024) void gres_bwd_rows_kernel(GatedResBwdArgs a, float* __restrict__ stats) {
    __shared__ float red[2 * 2 * 16];
    const int64_t t = blockIdx.x;
    const int c = threadIdx.x;
    const int C = a.C;
    const bool in = c < (C >> 3);
    const int m0 = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
    const bool mok = m0 >= 0 && m0 < a.n_rows;      // a row outside the table reads zeros
    const int64_t m = mok ? m0 : 0;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t mrow_bytes = mok ? row_bytes : 0u;
    const uint32_t off = 16u * uint32_t(c);
    float xv[8], ov[8], gv[8], dy[8], y[8];
    unpack8(bload16(make_rsrc(a.x + t * C, row_bytes), off, 0), xv);
    unpack8(bload16(make_rsrc(a.o + t * C, row_bytes), off, 0), ov);
    unpack8(bload16(make_rsrc(a.gate + m * C, mrow_bytes), off, 0), gv);
    unpack8(a.dy != nullptr ? bload16(make_rsrc(a.dy + t * C, row_bytes), off, 0) : u32x4_t{}, dy);
    u32x4_t pz = {0u, 0u, 0u, 0u}, ps2 = {0u, 0u, 0u, 0u};
    if constexpr (FUSED) {
        pz = bload16(make_rsrc(a.dz + t * C, row_bytes), off, 0);
        ps2 = bload16(make_rsrc(a.scale2 + m * C, mrow_bytes), off, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = xv[j] + gv[j] * ov[j];
    if constexpr (FUSED) {
        const float invC = 1.0f / float(C);
        float s[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) s[0] += y[j];        // chunks past the row hold y = 0
        wg_sum<2>(s, red, 0);
        const float mu = s[0] * invC;
        float v[2] = {0.f, 0.f};
        if (in)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[0] += (y[j] - mu) * (y[j] - mu);
        wg_sum<2>(v, red, 1);
        const float rs = rsqrtf(v[0] * invC + a.eps);
        float dz[8], s2[8], yh[8], g2[8];
        unpack8(pz, dz);
        unpack8(ps2, s2);
        float ab[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            yh[j] = (y[j] - mu) * rs;
            g2[j] = dz[j] * (1.0f + s2[j]);
            ab[0] += g2[j];
            ab[1] += g2[j] * yh[j];
        }
        wg_sum<2>(ab, red, 0);
        const float ma = ab[0] * invC, mb = ab[1] * invC;
#pragma unroll
        for (int j = 0; j < 8; ++j) dy[j] += (g2[j] - ma - yh[j] * mb) * rs;
        if (c == 0) *reinterpret_cast<f32x4_t*>(stats + 4 * t) = f32x4_t{mu, rs, ma, mb};
    }
    float dov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dov[j] = gv[j] * dy[j];
    bstore16(make_rsrc(a.dx + t * C, row_bytes), off, 0, pack8(dy));
    bstore16(make_rsrc(a.dout + t * C, row_bytes), off, 0, pack8(dov));
}

template <bool FUSED>
__global__ __launch_bounds__(64) void gres_bwd_sums_kernel(GatedResBwdArgs a, const float* __restrict__ stats,
                                                           int32_t* __restrict__ tags, float* __restrict__ slots) {
    constexpr int NA = FUSED ? 3 : 1;
    const int lane = threadIdx.x;
    const int C = a.C;
    const int c = blockIdx.y * kWave + lane;
    const bool live = c < (C >> 3);
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t voff = 16u * uint32_t(c);
    const int64_t t_begin = int64_t(blockIdx.x) * kSumRun;
    const int64_t t_end = t_begin + kSumRun < a.T ? t_begin + kSumRun : a.T;
    float* const outs[3] = {a.dgate, a.dshift2, a.dscale2};
    float sm[NA][8];
#pragma unroll
    for (int k = 0; k < NA; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) sm[k][j] = 0.f;
    int cur = -1;
    float gv[8], s2[8];
    auto flush = [&](int row) {
        if (row < 0 || row >= a.n_rows || !live) return;
#pragma unroll
        for (int k = 0; k < NA; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                atomic_add_f32(outs[k] + int64_t(row) * C + 8 * c + j, sm[k][j]);
                sm[k][j] = 0.f;
            }
    };
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            flush(cur);
            cur = m;
            const bool mok = m >= 0 && m < a.n_rows;
            const int64_t mm = mok ? m : 0;
            unpack8(bload16(make_rsrc(a.gate + mm * C, mok ? row_bytes : 0u), voff, 0), gv);
            if constexpr (FUSED) unpack8(bload16(make_rsrc(a.scale2 + mm * C, mok ? row_bytes : 0u), voff, 0), s2);
        }
        float xv[8], ov[8], dy[8], dz[8];
        unpack8(bload16(make_rsrc(a.x + t * C, row_bytes), voff, 0), xv);
        unpack8(bload16(make_rsrc(a.o + t * C, row_bytes), voff, 0), ov);
        unpack8(a.dy != nullptr ? bload16(make_rsrc(a.dy + t * C, row_bytes), voff, 0) : u32x4_t{}, dy);
        f32x4_t st = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FUSED) {
            unpack8(bload16(make_rsrc(a.dz + t * C, row_bytes), voff, 0), dz);
            st = *reinterpret_cast<const f32x4_t*>(stats + 4 * t);   // mu, rs, mean g2, mean g2 yh
        }
        if (m < 0 || m >= a.n_rows) continue;    // a row outside the table adds nothing
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float dyt = dy[j];
            if constexpr (FUSED) {
                const float yh = (xv[j] + gv[j] * ov[j] - st[0]) * st[1];
                dyt += (dz[j] * (1.0f + s2[j]) - st[2] - yh * st[3]) * st[1];
                sm[1][j] += dz[j];
                sm[2][j] += dz[j] * yh;
            }
            sm[0][j] += dyt * ov[j];
        }
    }
    float* slot = slots + int64_t(blockIdx.x) * NA * C;
    if (live)
#pragma unroll
        for (int k = 0; k < NA; ++k) {
            *reinterpret_cast<f32x4_t*>(slot + k * C + 8 * c) = f32x4_t{sm[k][0], sm[k][1], sm[k][2], sm[k][3]};
            *reinterpret_cast<f32x4_t*>(slot + k * C + 8 * c + 4) = f32x4_t{sm[k][4], sm[k][5], sm[k][6], sm[k][7]};
        }
    if (blockIdx.y == 0 && lane == 0) tags[blockIdx.x] = cur >= 0 && cur < a.n_rows ? cur : -1;
}

}  // namespace

size_t elementwise_bwd_workspace_bytes(int64_t T, int32_t C, int32_t n_arrays) {
    const int64_t Tn = T < 0 ? 0 : T;
    const int64_t ns = n_slots_for(Tn);
    // slots of kRun tokens (the single-kernel form), plus 16 bytes of row
    // statistics per token; the two-kernel form's fewer, larger-run slots and
    // its statistics fit the same bytes
    return slot_tags_bytes(ns) + size_t(ns) * size_t(n_arrays) * size_t(C) * 4 + size_t(Tn) * 16;
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
        const hipError_t e = zero_f32(a.dshift, a.dscale, nullptr, int64_t(a.n_rows) * C, stream);
        if (e != hipSuccess) return e;
    }
    if (a.T == 0) return hipSuccess;
    const int nch_w = (C / 8 + kWave - 1) / kWave;     // 16-byte chunks per lane of a row
    if (nch_w > 6) {
        hipLaunchKernelGGL(modulate_rope_bwd_kernel, dim3(unsigned(n_slots_for(a.T))), dim3(block_threads(C)), 0,
                           stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !mod) return e;
        return reduce_slots<2>(a.workspace, a.T, C, a.dshift, a.dscale, nullptr, stream);
    }
    // two kernels: workspace = tags, slots of kSumRun tokens, then the rows'
    // statistics (4 floats per token); it fits the size the single kernel's
    // slots need (C >= 64)
    const int64_t ns = sum_slots_for(a.T);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* tags = reinterpret_cast<int32_t*>(ws);
    float* slots = reinterpret_cast<float*>(ws + slot_tags_bytes(ns));
    float* stats = slots + ns * 2 * C;
    const dim3 grid_a(unsigned((a.T + kRowsTokens - 1) / kRowsTokens));
    switch (nch_w) {
        case 1: hipLaunchKernelGGL(modrope_bwd_dx_kernel<1>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 2: hipLaunchKernelGGL(modrope_bwd_dx_kernel<2>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 3: hipLaunchKernelGGL(modrope_bwd_dx_kernel<3>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 4: hipLaunchKernelGGL(modrope_bwd_dx_kernel<4>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 5: hipLaunchKernelGGL(modrope_bwd_dx_kernel<5>, grid_a, dim3(256), 0, stream, a, stats); break;
        default: hipLaunchKernelGGL(modrope_bwd_dx_kernel<6>, grid_a, dim3(256), 0, stream, a, stats); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !mod) return e;
    hipLaunchKernelGGL(modrope_bwd_sums_kernel, dim3(unsigned(ns), unsigned((C / 8 + kWave - 1) / kWave)), dim3(64),
                       0, stream, a, stats, tags, slots);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 grid(unsigned((ns + kSlotGroup - 1) / kSlotGroup), unsigned((C + 255) / 256));
    hipLaunchKernelGGL(slot_reduce_kernel<2>, grid, dim3(256), 0, stream, tags, slots, ns, C, a.dshift, a.dscale,
                       nullptr);
    return hipGetLastError();
}

hipError_t launch_gated_residual_bwd(const GatedResBwdArgs& a, hipStream_t stream) {
    const int64_t n = int64_t(a.n_rows) * a.C;
    const bool fused = a.dz != nullptr;
    hipError_t e = zero_f32(a.dgate, fused ? a.dshift2 : nullptr, fused ? a.dscale2 : nullptr, n, stream);
    if (e != hipSuccess) return e;
    if (a.T == 0) return hipSuccess;
    // workspace: tags, slots of kSumRun tokens (1 or 3 arrays), then the rows'
    // statistics (4 floats per token); it fits the size the query returns
    const int na = fused ? 3 : 1;
    const int64_t ns = sum_slots_for(a.T);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    int32_t* tags = reinterpret_cast<int32_t*>(ws);
    float* slots = reinterpret_cast<float*>(ws + slot_tags_bytes(ns));
    float* stats = slots + ns * na * a.C;
    const dim3 grid_b(unsigned(ns), unsigned((a.C / 8 + kWave - 1) / kWave));
    if (fused) {
        hipLaunchKernelGGL(gres_bwd_rows_kernel<true>, dim3(unsigned(a.T)), dim3(block_threads(a.C)), 0, stream, a,
                           stats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(gres_bwd_sums_kernel<true>, grid_b, dim3(64), 0, stream, a, stats, tags, slots);
    } else {
        hipLaunchKernelGGL(gres_bwd_rows_kernel<false>, dim3(unsigned(a.T)), dim3(block_threads(a.C)), 0, stream, a,
                           stats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(gres_bwd_sums_kernel<false>, grid_b, dim3(64), 0, stream, a, stats, tags, slots);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 grid(unsigned((ns + kSlotGroup - 1) / kSlotGroup), unsigned((a.C + 255) / 256));
    if (fused)
        hipLaunchKernelGGL(slot_reduce_kernel<3>, grid, dim3(256), 0, stream, tags, slots, ns, a.C, a.dgate,
                           a.dshift2, a.dscale2);
    else
        hipLaunchKernelGGL(slot_reduce_kernel<1>, grid, dim3(256), 0, stream, tags, slots, ns, a.C, a.dgate,
                           nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace mf
