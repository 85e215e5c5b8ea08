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
//    (4 16-byte loads), transposes the 4x8 bf16 block with byte permutes and
//    writes 8 x 8 bytes.  LDS layouts are bank-conflict free for the 16 lanes
//    a 16-byte access serves per cycle (32 lanes for 8-byte writes) over 64
//    banks, by padding rows (K: 256 -> 272 bytes, V^T: 128 -> 144 bytes)
//    rather than swizzling, so all operand addresses are affine.
//  * Full tiles run an unguarded path; only the ragged last tile of a
//    sequence masks keys and zero-fills its loads.
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
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kInlineSeqs = 64;  // packs up to this many sequences schedule in-kernel

template <int D>
struct Tile {
    static constexpr int KK = D / 16;            // QK^T MFMA steps along d
    static constexpr int EB = D / 32;            // 32-wide blocks of the output dim
    static constexpr int KCH = D / 8;            // 16-byte chunks per K row
    // K rows padded by one 16-byte unit: the 16 lanes one LDS cycle serves
    // (rows r..r+15, same chunk) then start 17 units apart, i.e. on 16
    // distinct 4-bank groups of the 64 banks, and every MFMA operand address
    // is the lane's base plus a compile-time offset.
    static constexpr int K_ROW_BYTES = D * 2 + 16;
    static constexpr int K_BYTES = kBN * K_ROW_BYTES;
    // V^T rows: 64 keys = 128 bytes (8 units of 16 bytes) padded to 144, so
    // that rows e and e+1 start 36 banks apart.
    static constexpr int VT_ROW_BYTES = kBN * 2 + 16;
    static constexpr int VT_BYTES = D * VT_ROW_BYTES;
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
    int n_seq;
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
    // Packs of up to kInlineSeqs sequences are scheduled here, by every
    // workgroup (cheaper than a prologue launch); larger ones read the
    // schedule the prologue kernel wrote into the workspace.
    __shared__ int32_t sched[3 * kInlineSeqs + 2];
    const int w = xcd_remap(blockIdx.x);
    const int n = p.n_seq;
    const int32_t* order;
    const int32_t* tiles;
    const int32_t* start;
    if (n <= kInlineSeqs) {
        int32_t* s_order = sched;
        int32_t* s_tiles = sched + kInlineSeqs;
        int32_t* s_start = sched + 2 * kInlineSeqs;
        if (threadIdx.x < 64) {
            const int sidx = threadIdx.x;
            const int Ls = sidx < n ? p.cu[sidx + 1] - p.cu[sidx] : -1;
            int rank = 0;
            for (int i = 0; i < n; ++i) {
                const int Li = p.cu[i + 1] - p.cu[i];
                rank += (Li > Ls) || (Li == Ls && i < sidx);
            }
            if (sidx < n) {
                s_order[rank] = sidx;
                s_tiles[rank] = (Ls + kBM - 1) / kBM;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int acc = 0;
            for (int r = 0; r < n; ++r) {
                s_start[r] = acc;
                acc += s_tiles[r] * p.H;
            }
            s_start[n] = acc;
            sched[3 * kInlineSeqs + 1] = acc;
        }
        __syncthreads();
        order = s_order;
        tiles = s_tiles;
        start = s_start;
        if (w >= sched[3 * kInlineSeqs + 1]) return;
    } else {
        if (w >= p.ws[0]) return;
        order = p.ws + 2;
        tiles = p.ws + 2 + n;
        start = p.ws + 2 + 2 * n;
    }
    int lo = 0, hi = n - 1;            // last rank with start[rank] <= w
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= w) lo = mid; else hi = mid - 1;
    }
    // The decoded unit is the same for every lane; say so, so that the
    // buffer resources and offsets below live in scalar registers.
    const int seq = __builtin_amdgcn_readfirstlane(order[lo]);
    const int nt = __builtin_amdgcn_readfirstlane(tiles[lo]);
    const int local = w - __builtin_amdgcn_readfirstlane(start[lo]);
    const int head = local / nt;
    const int qtile = local - head * nt;
    const int64_t tok0 = __builtin_amdgcn_readfirstlane(p.cu[seq]);
    const int L = __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int64_t ld = p.ld_qkv;

    // Buffer resources over this sequence's rows of the head: loads of rows
    // at or past L return zeros (ragged q-tile and last K/V tile).
    const uint64_t seq_bytes = uint64_t(L) * uint64_t(ld) * 2u;
    const int64_t head_off = (tok0 * ld + int64_t(head) * D);
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + head_off, seq_bytes);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + head_off, seq_bytes);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + head_off, seq_bytes);
    const uint32_t row_bytes = uint32_t(ld) * 2u;

    // ---- Q^T fragments (B operand), kept in registers -------------------
    const int qrow = qtile * kBM + wave * 32 + l32;    // row inside the sequence
    bf16x8_t qf[TL::KK];
    {
        const uint32_t qoff = uint32_t(qrow) * row_bytes + 16u * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, qoff, 32u * kk));
    }

    // ---- per-thread K/V load offsets and LDS addresses --------------------
    // K: thread -> (row k_row0 + 16*i, 16-byte chunk k_chunk).
    const int k_chunk = tid % TL::KCH;
    const int k_row0 = tid / TL::KCH;
    // V: thread -> (4-key group v_kg, 8-dim chunk v_ec); key group fastest so
    // the 32 lanes of one LDS write cycle cover two whole V^T rows 8 apart.
    const int v_kg = tid % (kBN / 4);
    const int v_ec = tid / (kBN / 4);
    const bool v_active = (TL::V_THREADS == kThreads) || tid < TL::V_THREADS;
    const uint32_t k_voff = uint32_t(k_row0) * row_bytes + 16u * k_chunk;
    const uint32_t v_voff = uint32_t(4 * v_kg) * row_bytes + 16u * v_ec;
    // LDS byte offsets inside one buffer
    const int k_wr = k_row0 * TL::K_ROW_BYTES + k_chunk * 16;
    const int v_wr = (8 * v_ec) * TL::VT_ROW_BYTES + (2 * (v_kg >> 2) + (v_kg & 1)) * 16 +
                     ((v_kg >> 1) & 1) * 8;
    const int k_rd = l32 * TL::K_ROW_BYTES + hlf * 16;                    // + b*32 rows + kk*32 B
    const int v_rd = TL::K_BYTES + l32 * TL::VT_ROW_BYTES + hlf * 16;     // + m*32 rows + cc*32 B

    u32x4_t kreg[TL::K_PASSES];
    u32x4_t vreg[4];

    // Global -> registers for the tile starting at key kv0 (rows past the end
    // of the sequence read as zeros).
    auto gload = [&](int kv0) {
        const uint32_t base = uint32_t(kv0) * row_bytes;
#pragma unroll
        for (int i = 0; i < TL::K_PASSES; ++i)
            kreg[i] = bload16(k_rs, k_voff, base + uint32_t(i * TL::K_ROWS_PER_PASS) * row_bytes);
        if (v_active) {
#pragma unroll
            for (int r = 0; r < 4; ++r) vreg[r] = bload16(v_rs, v_voff, base + uint32_t(r) * row_bytes);
        }
    };

    // Registers -> LDS buffer `buf`; V is transposed on the way (4 keys x 8
    // dims -> 8 rows of V^T, 4 keys each, in the MFMA key order).
    auto swrite = [&](int buf) {
        unsigned char* b = smem + buf * TL::BUF_BYTES;
#pragma unroll
        for (int i = 0; i < TL::K_PASSES; ++i)
            *reinterpret_cast<u32x4_t*>(b + k_wr + i * TL::K_ROWS_PER_PASS * TL::K_ROW_BYTES) = kreg[i];
        if (v_active) {
            unsigned char* vt = b + TL::K_BYTES + v_wr;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int wd = i >> 1;
                u32x2_t val;
                if ((i & 1) == 0) {
                    val[0] = lo_pair(vreg[0][wd], vreg[1][wd]);
                    val[1] = lo_pair(vreg[2][wd], vreg[3][wd]);
                } else {
                    val[0] = hi_pair(vreg[0][wd], vreg[1][wd]);
                    val[1] = hi_pair(vreg[2][wd], vreg[3][wd]);
                }
                *reinterpret_cast<u32x2_t*>(vt + i * TL::VT_ROW_BYTES) = val;
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
    const int nfull = L / kBN;                     // tiles needing no key mask

    // One K/V tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  `cur` is the
    // LDS buffer holding this tile; the next tile (if any) is fetched into
    // registers at the start and stored into the other buffer at the end.
    auto step = [&](int it, const int cur, bool masked) {
        const unsigned char* b = smem + cur * TL::BUF_BYTES;
        const int nxt = it + 1;
        if (nxt < nkv) gload(nxt * kBN);

        f32x16_t s[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[bb][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < TL::KK; ++kk) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
                    b + k_rd + bb * 32 * TL::K_ROW_BYTES + kk * 32);
                s[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[bb], 0, 0, 0);
            }
        }

        if (masked) {
            const int kv0 = it * kBN;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * bb + 8 * (r >> 2) + 4 * hlf + (r & 3);
                    if (key >= L) s[bb][r] = -INFINITY;
                }
        }

        // Online softmax for this lane's query row.  The exponentials use a
        // reference max m_run that is only raised when a row's block max
        // exceeds it by more than kRescaleLog2 (so p <= 2^kRescaleLog2);
        // numerator and denominator share m_run, so the result is the same
        // softmax, and the output accumulator is rescaled only on those
        // (rare, wave-uniform) occasions.
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = (bb == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, s[bb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
        const bool raise = mx > m_run + kRescaleLog2;
        if (__any(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = exp2f(m_run - m_new);      // 1 where not raised, 0 at start
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int m = 0; m < TL::EB; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
        }
        float lsum = 0.f;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], c, -m_run));
                s[bb][r] = e;
                lsum += e;
            }
        l_run += lsum;

        // P^T fragments (bf16) for the four 16-key chunks.
        bf16x8_t pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int bb = cc >> 1;
            const int r0 = 8 * (cc & 1);
            u32x4_t u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(s[bb][r0 + 2 * i], s[bb][r0 + 2 * i + 1]);
            pf[cc] = __builtin_bit_cast(bf16x8_t, u);
        }

        // O^T += V^T P^T
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(
                    b + v_rd + m * 32 * TL::VT_ROW_BYTES + cc * 32);
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], oacc[m], 0, 0, 0);
            }

        if (nxt < nkv) swrite(cur ^ 1);
        __syncthreads();
    };

    gload(0);
    swrite(0);
    __syncthreads();
    int it = 0;
    for (; it + 2 <= nfull; it += 2) {       // unrolled pair: buffers 0 then 1
        step(it, 0, false);
        step(it + 1, 1, false);
    }
    if (it < nfull) {
        step(it, 0, false);
        ++it;
    }
    if (it < nkv) step(it, it & 1, true);

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
    if (a.n_seq > kInlineSeqs) {
        hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seq, a.H, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    KParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
    p.cu = a.cu_seqlens; p.ws = ws; p.n_seq = a.n_seq; p.T = a.T;
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
