// Text-encoder variant of the hot path (gfx950): per-head RMS normalisation +
// rotary embedding of q and k, and causal attention with grouped key/value
// heads over packed prompts.
//
// The pages fuse the normalisation and rotary-embedding chains inside the
// frozen Qwen3-VL text encoder's blocks as in the backbone (picx.dev summary
// of Mage-Flow, Methodology > Training Infrastructure; gist.science "Resumo
// Tecnico: Mage-Flow", Metodologia > 3 > Kernels Fundidos); its prompts
// condition the backbone and are packed like its samples (picx.dev,
// Methodology > Native-Resolution MMDiT).
//
//   q'[t][h] = RoPE_p(q[t][h] / sqrt(mean(q[t][h]^2) + eps) * wq),  k' alike
//   O[i][h]  = softmax_j<=i(tau q'_i k'_j) v_j   inside each prompt,
//              key/value head h / (Hq / Hkv)
// with p the token's index inside its prompt and RoPE on adjacent pairs.
//
// Design (MI355X, CDNA4):
//  * qknorm_rope_kernel: one wavefront per token; lane l owns the 16-byte
//    chunks l, l+64, ... of the q and k rows, all at the same in-head offset
//    e0 = 8 (l mod D/8), so the four rotation angles of a lane are computed
//    once per token and a head's sum of squares is a reduction over the D/8
//    lanes that hold it (DPP inside a 16-lane row).
//  * attn_causal_kernel<D>: a work unit is 128 queries of one query head of
//    one prompt (4 wavefronts, 32 queries each; two workgroups per CU), a
//    one-workgroup prologue numbers the units.  The unit walks the key tiles
//    of 64 up to its diagonal only; K and V tiles of the grouped key/value
//    head are staged through registers one tile ahead into two LDS buffers.
//    Per tile a wavefront computes S^T = K Q^T (each lane: one query, 16 keys
//    per 32-key block), masks keys past the query or past the prompt on the
//    tiles that reach them, runs the online softmax with a lazily raised
//    reference max, and accumulates O^T += V^T P^T with V^T read transposed
//    from LDS (ds_read_b64_tr_b16) and P^T rounded to bf16 in registers.
#include <cmath>
#include <type_traits>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

// Sum over the n lanes (n = 8 or 16, aligned) that hold one head: DPP
// swaps inside quads, then mirrors inside 8 and 16 lanes.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (N == 16) v += dpp<0x140>(v);   // row_mirror
    return v;
}

template <int D, int NCQ, int NCK>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(QkNormRopeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    constexpr int kCh = D / 8;                    // chunks per head
    const int e0 = 8 * (lane % kCh);
    const double p = double(a.pos[t]);
    float cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double turns = p * a.theta_turns[e0 / 2 + j];
        const float f = float(turns - rint(turns));
        sn[j] = __builtin_amdgcn_sinf(f);
        cs[j] = __builtin_amdgcn_cosf(f);
    }
    float wq[8], wk[8];
    unpack8(ld16(a.wq + e0), wq);
    unpack8(ld16(a.wk + e0), wk);
    auto row = [&](const uint16_t* in, uint16_t* out, int C, const float* w, auto ncc) {
        constexpr int NC = decltype(ncc)::value;
        const uint32_t bytes = uint32_t(C) * 2u;
        const __amdgpu_buffer_rsrc_t in_rs = make_rsrc(in, bytes);
        const __amdgpu_buffer_rsrc_t out_rs = make_rsrc(out, bytes);
        u32x4_t px[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) px[i] = bload16(in_rs, 16u * uint32_t(lane + 64 * i), 0);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            float x[8];
            unpack8(px[i], x);
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
            const float r = rsqrtf(group_sum<kCh>(ss) * (1.0f / D) + a.eps);
            float y[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x0 = x[2 * j] * r * w[2 * j], x1 = x[2 * j + 1] * r * w[2 * j + 1];
                y[2 * j] = x0 * cs[j] - x1 * sn[j];
                y[2 * j + 1] = x0 * sn[j] + x1 * cs[j];
            }
            bstore16(out_rs, 16u * uint32_t(lane + 64 * i), 0, pack8(y));
        }
    };
    row(a.q_in + t * a.ld_q, a.q_out + t * a.ld_qo, a.Hq * D, wq, std::integral_constant<int, NCQ>{});
    row(a.k_in + t * a.ld_k, a.k_out + t * a.ld_ko, a.Hkv * D, wk, std::integral_constant<int, NCK>{});
}

template <int D, int NCQ>
hipError_t launch_qknorm_k(const QkNormRopeArgs& a, hipStream_t stream) {
    const int nck = (a.Hkv * D / 8 + 63) / 64;
    const unsigned blocks = unsigned((a.T + 3) / 4);
    if (nck <= 1) { hipLaunchKernelGGL((qknorm_rope_kernel<D, NCQ, 1>), dim3(blocks), dim3(256), 0, stream, a); }
    else if (nck <= 2) { hipLaunchKernelGGL((qknorm_rope_kernel<D, NCQ, 2>), dim3(blocks), dim3(256), 0, stream, a); }
    else if (nck <= 4) { hipLaunchKernelGGL((qknorm_rope_kernel<D, NCQ, 4>), dim3(blocks), dim3(256), 0, stream, a); }
    else if (nck <= 8) { hipLaunchKernelGGL((qknorm_rope_kernel<D, NCQ, 8>), dim3(blocks), dim3(256), 0, stream, a); }
    else { hipLaunchKernelGGL((qknorm_rope_kernel<D, NCQ, 16>), dim3(blocks), dim3(256), 0, stream, a); }
    return hipGetLastError();
}

template <int D>
hipError_t launch_qknorm_d(const QkNormRopeArgs& a, hipStream_t stream) {
    const int ncq = (a.Hq * D / 8 + 63) / 64;
    if (ncq <= 1) return launch_qknorm_k<D, 1>(a, stream);
    if (ncq <= 2) return launch_qknorm_k<D, 2>(a, stream);
    if (ncq <= 4) return launch_qknorm_k<D, 4>(a, stream);
    if (ncq <= 8) return launch_qknorm_k<D, 8>(a, stream);
    return launch_qknorm_k<D, 16>(a, stream);
}

// ---------------------------------------------------------------------------
// Causal attention with grouped key/value heads
// ---------------------------------------------------------------------------
constexpr int kCW = 4;                 // wavefronts per workgroup
constexpr int kCM = 32 * kCW;          // queries per work unit
constexpr int kCN = 64;                // keys per tile
constexpr float kRescale = 8.0f;       // lazy-rescale threshold (log2 units)

template <int D>
struct CT {
    static constexpr int KK = D / 16;
    static constexpr int EB = D / 32;
    static constexpr int KCH = D / 8;
    static constexpr int K_ROW = 16 * (KCH + 1);     // conflict-free 16-byte row reads
    static constexpr int V_ROW = 16 * (KCH + 4);     // conflict-free transposed reads
    static constexpr int K_BYTES = kCN * K_ROW;
    static constexpr int V_BYTES = kCN * V_ROW;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int STAGE_CH = kCN * KCH / (64 * kCW);   // 16-byte chunks per thread per tile
    static_assert(kCN * KCH % (64 * kCW) == 0, "whole staging chunks");
};

// Per-prompt query-tile counts and their prefix sums (one workgroup).
__global__ __launch_bounds__(256) void causal_tiles_kernel(const int32_t* __restrict__ cu, int n,
                                                           int64_t* __restrict__ pre) {
    __shared__ int64_t part[256];
    const int tid = threadIdx.x;
    const int per = (n + 255) / 256;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    int64_t acc = 0;
    for (int s = s0; s < s1; ++s) acc += (cu[s + 1] - cu[s] + kCM - 1) / kCM;
    part[tid] = acc;
    __syncthreads();
    if (tid == 0) {
        int64_t r = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t v = part[i];
            part[i] = r;
            r += v;
        }
        pre[n] = r;
    }
    __syncthreads();
    int64_t b = part[tid];
    for (int s = s0; s < s1; ++s) {
        pre[s] = b;
        b += (cu[s + 1] - cu[s] + kCM - 1) / kCM;
    }
}

// Work unit -> (prompt, query head, tile); units of prompt s are
// [pre[s] H, pre[s+1] H), head-major.  False past the last unit.
__device__ bool causal_unit(const int64_t* pre, int n, int H, int64_t unit, int& s, int& h, int& tile) {
    if (unit >= pre[n] * H) return false;
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] * H <= unit) lo = mid; else hi = mid - 1;
    }
    const int64_t local = unit - pre[lo] * H;
    const int64_t tiles = pre[lo + 1] - pre[lo];
    s = lo;
    h = int(local / tiles);
    tile = int(local - int64_t(h) * tiles);
    return true;
}

__device__ __forceinline__ float half_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct CausalParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* cu;
    const int64_t* pre;
    int n_seq, Hq, Hkv;
    int64_t T, ld_q, ld_kv, ld_o;
    float c;            // softmax scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(64 * kCW) void attn_causal_kernel(CausalParams p) {
    using TL = CT<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int seq, head, tile;
    if (!causal_unit(p.pre, p.n_seq, p.Hq, blockIdx.x, seq, head, tile)) return;
    seq = __builtin_amdgcn_readfirstlane(seq);
    head = __builtin_amdgcn_readfirstlane(head);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const int kvh = head / (p.Hq / p.Hkv);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int64_t tok0 = __builtin_amdgcn_readfirstlane(p.cu[seq]);
    const int L = __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);
    const uint32_t qrow = uint32_t(p.ld_q) * 2u, kvrow = uint32_t(p.ld_kv) * 2u;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + tok0 * p.ld_q + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + tok0 * p.ld_kv + int64_t(kvh) * D, uint64_t(L) * kvrow);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + tok0 * p.ld_kv + int64_t(kvh) * D, uint64_t(L) * kvrow);

    // the wavefront's 32 queries (B operand of S^T = K Q^T)
    const int q0 = tile * kCM + wave * 32;
    const int qi = q0 + l32;                     // this lane's query, inside the prompt
    bf16x8_t qf[TL::KK];
    {
        const uint32_t off = uint32_t(qi) * qrow + 16u * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk) qf[kk] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, off, 32u * kk));
    }
    // key tiles up to the unit's last query (and the prompt's end)
    const int last_q = min(L - 1, tile * kCM + kCM - 1);
    const int nt = last_q / kCN + 1;

    u32x4_t sk[TL::STAGE_CH], sv[TL::STAGE_CH];
    auto st_row = [&](int j) { return (tid + 64 * kCW * j) / TL::KCH; };
    auto st_col = [&](int j) { return (tid + 64 * kCW * j) % TL::KCH; };
    auto stage_load = [&](int t) {
#pragma unroll
        for (int j = 0; j < TL::STAGE_CH; ++j) {
            const uint32_t off = uint32_t(t * kCN + st_row(j)) * kvrow + 16u * st_col(j);
            sk[j] = bload16(k_rs, off, 0);
            sv[j] = bload16(v_rs, off, 0);
        }
    };
    auto stage_store = [&](int b) {
        unsigned char* base = smem + b * TL::STAGE;
#pragma unroll
        for (int j = 0; j < TL::STAGE_CH; ++j) {
            *reinterpret_cast<u32x4_t*>(base + st_row(j) * TL::K_ROW + 16 * st_col(j)) = sk[j];
            *reinterpret_cast<u32x4_t*>(base + TL::K_BYTES + st_row(j) * TL::V_ROW + 16 * st_col(j)) = sv[j];
        }
    };

    f32x16_t oacc[TL::EB];
#pragma unroll
    for (int m = 0; m < TL::EB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.c;
    const int k_rd = l32 * TL::K_ROW + hlf * 16;
    const int v_rd = (4 * hlf + ((lane & 15) >> 2)) * TL::V_ROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    stage_load(0);
    stage_store(0);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
        if (t + 1 < nt) stage_load(t + 1);
        const unsigned char* kt = smem + (t & 1) * TL::STAGE;
        const unsigned char* vt = kt + TL::K_BYTES;
        // S^T = K Q^T: two 32-key blocks (lane: query qi, register r: key
        // 32 b + 8 (r/4) + 4 h + r%4 of the tile)
        f32x16_t s[2];
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + k_rd + b * 32 * TL::K_ROW + kk * 32);
                s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], kk == 0 ? f32x16_t{} : s[b], 0, 0, 0);
            }
        // keys past the query (causal) or past the prompt: only tiles that
        // reach the wavefront's first query or the prompt's end
        if ((t + 1) * kCN - 1 > q0 || (t + 1) * kCN > L) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t * kCN + 32 * b + 8 * (r >> 2) + 4 * hlf + (r & 3);
                    if (key > qi || key >= L) s[b][r] = -INFINITY;
                }
        }
        // online softmax, reference max raised lazily (numerator and
        // denominator share it, so the result is the same softmax)
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = (b == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, s[b][r]);
        mx = half_max32(mx) * c;
        const bool raise = mx > m_run + kRescale;
        if (__any(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int m = 0; m < TL::EB; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
        }
        float lsum = 0.f;
        bf16x8_t pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int b = cc >> 1, r0 = 8 * (cc & 1);
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r0 + i], c, -m_run));
                lsum += e[i];
            }
            u32x4_t u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
            pf[cc] = __builtin_bit_cast(bf16x8_t, u);
        }
        l_run += lsum;
        // O^T += V^T P^T over the four 16-key chunks
#pragma unroll
        for (int j = 0; j < 4 * TL::EB; ++j) {
            const unsigned char* ad = vt + v_rd + (j / TL::EB) * 16 * TL::V_ROW + (j % TL::EB) * 64;
            const s16x4_t lo = lds_read_tr16_b64(ad);
            const s16x4_t hi = lds_read_tr16_b64(ad + 8 * TL::V_ROW);
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[j % TL::EB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j / TL::EB], oacc[j % TL::EB], 0, 0, 0);
        }
        // the other buffer was last read in step t-1, finished by everyone
        // before the barrier that opened step t
        if (t + 1 < nt) stage_store((t + 1) & 1);
        __syncthreads();
    }

    const float l_tot = half_sum32(l_run);
    if (qi < L) {
        const float inv = 1.0f / l_tot;
        uint16_t* op = p.o + (tok0 + qi) * p.ld_o + int64_t(head) * D + 4 * hlf;
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2_t val;
                val[0] = pack_bf16x2(oacc[m][4 * g] * inv, oacc[m][4 * g + 1] * inv);
                val[1] = pack_bf16x2(oacc[m][4 * g + 2] * inv, oacc[m][4 * g + 3] * inv);
                *reinterpret_cast<u32x2_t*>(op + 32 * m + 8 * g) = val;
            }
        if (p.lse != nullptr && hlf == 0) p.lse[int64_t(head) * p.T + tok0 + qi] = m_run * 0.69314718055994531f + logf(l_tot);
    }
}

template <int D>
hipError_t launch_causal_d(const CausalAttnArgs& a, hipStream_t stream) {
    CausalParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse; p.cu = a.cu_seqlens;
    p.pre = static_cast<const int64_t*>(a.workspace);
    p.n_seq = a.n_seq; p.Hq = a.Hq; p.Hkv = a.Hkv;
    p.T = a.T; p.ld_q = a.ld_q; p.ld_kv = a.ld_kv; p.ld_o = a.ld_o;
    p.c = a.softmax_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(causal_tiles_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seq,
                       static_cast<int64_t*>(a.workspace));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_causal_kernel<D>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, CT<D>::LDS);
    if (attr != hipSuccess) return attr;
    // upper bound of the unit count: sum_s ceil(L_s / kCM) <= T / kCM + n_seq
    const int64_t units = int64_t(a.Hq) * (a.T / kCM + a.n_seq);
    hipLaunchKernelGGL(attn_causal_kernel<D>, dim3(unsigned(units)), dim3(64 * kCW), CT<D>::LDS, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope(const QkNormRopeArgs& args, hipStream_t stream) {
    QkNormRopeArgs a = args;
    if (a.T == 0) return hipSuccess;
    for (int j = 0; j < a.D / 2; ++j)
        a.theta_turns[j] = std::pow(double(a.rope_base), -2.0 * j / double(a.D)) * 0.15915494309189535;
    return a.D == 128 ? launch_qknorm_d<128>(a, stream) : launch_qknorm_d<64>(a, stream);
}

size_t causal_attn_workspace_bytes(int32_t n_seq) {
    return size_t(n_seq < 0 ? 0 : n_seq + 1) * sizeof(int64_t);
}

hipError_t launch_varlen_attn_causal(const CausalAttnArgs& a, hipStream_t stream) {
    if (a.T == 0 || a.n_seq == 0) return hipSuccess;
    return a.D == 128 ? launch_causal_d<128>(a, stream) : launch_causal_d<64>(a, stream);
}

}  // namespace mf
