// Block-diagonal (varlen) joint softmax attention forward for gfx950.
//
// What it computes: for every packed sequence (delimited by cumulative
// offsets) and head, O = softmax(scale * Q K^T) V with no mask inside the
// sequence and nothing across sequences, plus the row log-sum-exp.  Sources:
// picx.dev summary of Mage-Flow, Methodology > Native-Resolution MMDiT
// (variable-length attention over packed samples with per-sample cumulative
// offsets; joint self-attention of text and image tokens); gist.science
// "Resumo Tecnico: Mage-Flow", Metodologia > 2. NR-MMDiT.
//
// Design (MI355X, CDNA4):
//  * Work unit = (sequence, head, 128-query tile).  A one-workgroup prologue
//    kernel orders the sequences longest first and writes the unit ranges
//    into the caller's workspace; the main grid maps blockIdx to units with
//    an XCD-aware permutation so that consecutive units (same sequence and
//    head, hence the same K/V) land on the same XCD and share its L2.
//  * 256 threads = 4 wavefronts; each wavefront owns 32 query rows.  The Q
//    rows live in VGPRs for the whole tile as MFMA B operands.
//  * K/V advance in 64-key tiles, double-buffered in LDS: the next tile's
//    global loads are issued before the current tile's MFMAs and written to
//    the other LDS buffer after them, one barrier per tile.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: every lane then holds 16 keys of one query
//    row, so the online-softmax max/sum need one cross-half exchange and
//    the rescale of the output accumulator is a per-lane scalar.
//  * The fp32 probabilities are rounded to bf16 in registers and used
//    directly as the B operand of O^T += V^T P^T: the MFMA accumulator
//    layout of S^T gives each lane keys {4h..4h+3, 8+4h..8+4h+3} of every
//    16-key chunk, so V^T is stored in LDS with that key order inside each
//    16-key chunk and read with one 16-byte access per MFMA.
//  * V is transposed on the way into LDS: each thread loads 4 keys x 8 dims
//    (4 coalesced 16-byte loads), transposes the 4x8 bf16 block with byte
//    permutes and writes 8 x 8 bytes.  K and V^T tiles use XOR swizzles of
//    their 16-byte units so that MFMA operand reads are bank-conflict free.
//  * exp2 with the softmax scale folded into one FMA (scale * log2 e);
//    all softmax state in fp32.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kXcds = 8;        // XCDs of an MI355X; blockIdx round-robins over them
constexpr int kXcdGroup = 8;    // consecutive work units kept on one XCD

template <int D>
struct Tile {
    static constexpr int KK = D / 16;            // QK^T MFMA steps along d
    static constexpr int EB = D / 32;            // 32-wide blocks of the output dim
    static constexpr int KCH = D / 8;            // 16-byte chunks per K row
    static constexpr int K_ROW_BYTES = D * 2;
    static constexpr int K_BYTES = kBN * D * 2;
    static constexpr int VT_ROW_BYTES = kBN * 2; // 128 bytes: 8 units of 16 bytes
    static constexpr int VT_BYTES = D * kBN * 2;
    static constexpr int BUF_BYTES = K_BYTES + VT_BYTES;
    static constexpr int K_ROWS_PER_PASS = kThreads / KCH;
    static constexpr int K_PASSES = kBN / K_ROWS_PER_PASS;
    static constexpr int V_THREADS = (D / 8) * (kBN / 4);   // 8 dims x 4 keys per thread
};

// Workspace layout (int32): [0] number of work units, [1] n_seq,
// [2 .. 2+n) sequence index by rank (longest first), [2+n .. 2+2n) q-tiles of
// that sequence, [2+2n .. 3+3n) first work unit of each rank (exclusive
// prefix over tiles*H, with the total at the end).
__global__ __launch_bounds__(256) void attn_schedule_kernel(const int32_t* __restrict__ cu, int n,
                                                            int H, int32_t* __restrict__ ws) {
    int32_t* order = ws + 2;
    int32_t* tiles = ws + 2 + n;
    int32_t* start = ws + 2 + 2 * n;
    for (int s = threadIdx.x; s < n; s += blockDim.x) {
        const int Ls = cu[s + 1] - cu[s];
        int rank = 0;
        for (int i = 0; i < n; ++i) {
            const int Li = cu[i + 1] - cu[i];
            rank += (Li > Ls) || (Li == Ls && i < s);
        }
        order[rank] = s;
        tiles[rank] = (Ls + kBM - 1) / kBM;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int r = 0; r < n; ++r) {
            start[r] = acc;
            acc += tiles[r] * H;
        }
        start[n] = acc;
        ws[0] = acc;
        ws[1] = n;
    }
}

__device__ __forceinline__ int xcd_remap(int b) {
    const int x = b % kXcds;
    const int tau = b / kXcds;
    return ((tau / kXcdGroup) * kXcds + x) * kXcdGroup + (tau % kXcdGroup);
}

struct KParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* cu;
    const int32_t* ws;
    int64_t T;
    int64_t ld_qkv, ld_o;
    int H;
    float scale_log2;   // softmax_scale * log2(e)
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    // low bf16 of a in the low half, low bf16 of b in the high half
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(KParams p) {
    using TL = Tile<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- decode the work unit -------------------------------------------
    const int w = xcd_remap(blockIdx.x);
    const int nwork = p.ws[0];
    if (w >= nwork) return;
    const int n = p.ws[1];
    const int32_t* order = p.ws + 2;
    const int32_t* tiles = p.ws + 2 + n;
    const int32_t* start = p.ws + 2 + 2 * n;
    int lo = 0, hi = n - 1;            // last rank with start[rank] <= w
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= w) lo = mid; else hi = mid - 1;
    }
    const int seq = order[lo];
    const int nt = tiles[lo];
    const int local = w - start[lo];
    const int head = local / nt;
    const int qtile = local - head * nt;
    const int64_t tok0 = p.cu[seq];
    const int L = p.cu[seq + 1] - p.cu[seq];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;

    // ---- Q^T fragments (B operand), kept in registers -------------------
    const int qrow = qtile * kBM + wave * 32 + l32;    // row inside the sequence
    bf16x8_t qf[TL::KK];
    {
        const uint16_t* qp = p.q + (tok0 + qrow) * p.ld_qkv + int64_t(head) * D + 8 * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk) {
            u32x4_t v = {0, 0, 0, 0};
            if (qrow < L) v = ld16(qp + 16 * kk);
            qf[kk] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    const uint16_t* kb = p.k + tok0 * p.ld_qkv + int64_t(head) * D;
    const uint16_t* vb = p.v + tok0 * p.ld_qkv + int64_t(head) * D;

    // K tile load mapping: thread -> (row, 16-byte chunk)
    const int k_chunk = tid % TL::KCH;
    const int k_row0 = tid / TL::KCH;
    // V tile load mapping: thread -> (4-key group, 8-dim chunk)
    const int v_ec = tid % (D / 8);
    const int v_kg = tid / (D / 8);
    const bool v_active = tid < TL::V_THREADS;

    u32x4_t kreg[TL::K_PASSES];
    u32x4_t vreg[4];

    auto gload = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < TL::K_PASSES; ++i) {
            const int r = kv0 + k_row0 + i * TL::K_ROWS_PER_PASS;
            u32x4_t v = {0, 0, 0, 0};
            if (r < L) v = ld16(kb + int64_t(r) * p.ld_qkv + 8 * k_chunk);
            kreg[i] = v;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kv0 + 4 * v_kg + r;
            u32x4_t v = {0, 0, 0, 0};
            if (v_active && key < L) v = ld16(vb + int64_t(key) * p.ld_qkv + 8 * v_ec);
            vreg[r] = v;
        }
    };

    auto swrite = [&](int buf) {
        unsigned char* kt = smem + buf * TL::BUF_BYTES;
        unsigned char* vt = kt + TL::K_BYTES;
#pragma unroll
        for (int i = 0; i < TL::K_PASSES; ++i) {
            const int r = k_row0 + i * TL::K_ROWS_PER_PASS;
            *reinterpret_cast<u32x4_t*>(kt + r * TL::K_ROW_BYTES + ((k_chunk ^ (r & 7)) << 4)) = kreg[i];
        }
        if (v_active) {
            // 4 keys x 8 dims -> for each dim, the 4 keys as one 8-byte write.
            const int q16 = v_kg >> 2;               // 16-key chunk
            const int wq = v_kg & 3;                 // which 4 keys inside it
            const int unit = 2 * q16 + (wq & 1);
            const int half = wq >> 1;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = 8 * v_ec + i;
                const int wd = i >> 1;
                u32x2_t val;
                if ((i & 1) == 0) {
                    val[0] = lo_pair(vreg[0][wd], vreg[1][wd]);
                    val[1] = lo_pair(vreg[2][wd], vreg[3][wd]);
                } else {
                    val[0] = hi_pair(vreg[0][wd], vreg[1][wd]);
                    val[1] = hi_pair(vreg[2][wd], vreg[3][wd]);
                }
                const int swz = (e + (e >> 3)) & 7;
                *reinterpret_cast<u32x2_t*>(vt + e * TL::VT_ROW_BYTES + ((unit ^ swz) << 4) + half * 8) = val;
            }
        }
    };

    f32x16_t oacc[TL::EB];
#pragma unroll
    for (int m = 0; m < TL::EB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = p.scale_log2;

    const int nkv = (L + kBN - 1) / kBN;
    gload(0);
    swrite(0);
    __syncthreads();

    for (int it = 0; it < nkv; ++it) {
        const int cur = it & 1;
        const unsigned char* kt = smem + cur * TL::BUF_BYTES;
        const unsigned char* vt = kt + TL::K_BYTES;
        if (it + 1 < nkv) gload((it + 1) * kBN);

        // S^T = K Q^T for keys [it*64, it*64+64): two 32-key blocks.
        f32x16_t s[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
            const int row = 32 * b + l32;
#pragma unroll
            for (int kk = 0; kk < TL::KK; ++kk) {
                const int ch = 2 * kk + hlf;
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
                    kt + row * TL::K_ROW_BYTES + ((ch ^ (row & 7)) << 4));
                s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[b], 0, 0, 0);
            }
        }

        // Mask keys past the end of the sequence (last tile only).
        if ((it + 1) * kBN > L) {
            const int kv0 = it * kBN;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * b + 8 * (r >> 2) + 4 * hlf + (r & 3);
                    if (key >= L) s[b][r] = -INFINITY;
                }
        }

        // Online softmax for this lane's query row.
        float mx = s[0][0];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -m_new));
                s[b][r] = e;
                lsum += e;
            }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;

        // P^T fragments (bf16) for the four 16-key chunks.
        bf16x8_t pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int b = cc >> 1;
            const int r0 = 8 * (cc & 1);
            u32x4_t u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(s[b][r0 + 2 * i], s[b][r0 + 2 * i + 1]);
            pf[cc] = __builtin_bit_cast(bf16x8_t, u);
        }

        // O^T += V^T P^T
#pragma unroll
        for (int m = 0; m < TL::EB; ++m) {
            const int e = 32 * m + l32;
            const int swz = (e + (e >> 3)) & 7;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int unit = 2 * cc + hlf;
                const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(
                    vt + e * TL::VT_ROW_BYTES + ((unit ^ swz) << 4));
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], oacc[m], 0, 0, 0);
            }
        }

        if (it + 1 < nkv) swrite(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if (qrow < L) {
        const float inv = 1.0f / l_tot;
        uint16_t* op = p.o + (tok0 + qrow) * p.ld_o + int64_t(head) * D + 4 * hlf;
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2_t val;
                val[0] = pack_bf16x2(oacc[m][4 * g] * inv, oacc[m][4 * g + 1] * inv);
                val[1] = pack_bf16x2(oacc[m][4 * g + 2] * inv, oacc[m][4 * g + 3] * inv);
                *reinterpret_cast<u32x2_t*>(op + 32 * m + 8 * g) = val;
            }
        if (p.lse != nullptr && hlf == 0)
            p.lse[int64_t(head) * p.T + tok0 + qrow] = m_run * 0.69314718055994531f + logf(l_tot);
    }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
    int32_t* ws = static_cast<int32_t*>(a.workspace);
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seq,
                       a.H, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
    p.cu = a.cu_seqlens; p.ws = ws; p.T = a.T;
    p.ld_qkv = a.ld_qkv; p.ld_o = a.ld_o; p.H = a.H;
    p.scale_log2 = a.softmax_scale * 1.4426950408889634f;
    // Upper bound of the work units: sum_s ceil(L_s/128) <= T/128 + n_seq.
    const int64_t units = int64_t(a.H) * ((a.T + kBM - 1) / kBM + a.n_seq);
    const int64_t quantum = int64_t(kXcds) * kXcdGroup;
    const int64_t grid = (units + quantum - 1) / quantum * quantum;
    const size_t smem = 2 * Tile<D>::BUF_BYTES;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_fwd_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(smem));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(unsigned(grid)), dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int32_t n_seq, int64_t /*T*/, int32_t /*H*/, int32_t /*D*/) {
    const size_t ints = 3 + 3 * size_t(n_seq < 0 ? 0 : n_seq);
    return (ints * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_varlen_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_d<128>(a, stream);
    return launch_d<64>(a, stream);
}

}  // namespace mf
