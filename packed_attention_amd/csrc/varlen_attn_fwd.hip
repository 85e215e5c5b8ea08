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
//  * Work unit = (sequence, head, 128-query tile).  Sequences are ordered
//    longest first (in-kernel for packs of up to 64 sequences, otherwise by a
//    one-workgroup prologue kernel writing into the caller's workspace), and
//    blockIdx maps to units through an XCD-aware permutation so consecutive
//    units (same sequence and head, hence the same K/V) share one XCD's L2.
//  * One workgroup of 8 wavefronts per CU (two per SIMD, 256 registers
//    each) sharing every K/V tile; each wavefront owns 32 query rows, held
//    in VGPRs as MFMA B operands for the whole tile.  Two waves per SIMD
//    because one wavefront alone cannot stream LDS operands fast enough to
//    feed its MFMAs (about 1 KiB per 32-cycle MFMA).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: every lane holds 16 keys of one query row, so
//    the online-softmax max/sum need one v_permlane32_swap and the rescale of
//    the output accumulator is a per-lane scalar.  The fp32 probabilities are
//    rounded to bf16 in registers and used directly as the B operand of
//    O^T += V^T P^T: V^T is stored in LDS with the key order that the S^T
//    accumulator layout gives each lane ({4h..4h+3, 8+4h..8+4h+3} of every
//    16-key chunk), read with one 16-byte access per MFMA.
//  * Per 64-key tile a wavefront runs S^T = K Q^T (2*D/16 MFMAs), the
//    online softmax (VALU), then O^T += V^T P^T (D/8 MFMAs); with two waves
//    per SIMD one wave's softmax runs while the other's MFMAs execute.
//    Operand fragments are read from LDS four MFMAs ahead, pinned with
//    sched_barrier so the scheduler does not sink them next to their use.
//  * K and V arrive by direct global->LDS buffer loads (no staging
//    registers, no LDS stores), double-buffered: tile t+1 is fetched while
//    tile t is consumed, one barrier per tile.  V stays row-major and is
//    read transposed (ds_read_b64_tr_b16) into the V^T operand.  Rows are
//    padded (K: 2D -> 2D+16 bytes, V: 2D -> 2D+64) so every LDS read cycle
//    hits distinct banks of the 64, with affine addresses.
//  * Q/K/V are read through raw buffer resources that end at the sequence's
//    last row, so ragged tiles read zeros without branches; only the last
//    tile of a sequence masks its scores.
//  * exp2 with the softmax scale folded into one FMA (scale * log2 e); the
//    reference max is raised lazily (only when a row max grows by more than
//    2^8), so the output accumulator is rarely rescaled; all softmax state
//    in fp32.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kWaves = 8;       // wavefronts per workgroup: 2 per SIMD
constexpr int kBM = 32 * kWaves; // query rows per workgroup (32 per wavefront)
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;        // XCDs of an MI355X; blockIdx round-robins over them
constexpr int kXcdGroup = 32;   // consecutive work units kept on one XCD (its 32 CUs)
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kInlineSeqs = 64;  // packs up to this many sequences schedule in-kernel
constexpr int kPrefetch = 4;     // MFMA operand fragments read ahead from LDS

template <int D>
struct Tile {
    static constexpr int KK = D / 16;            // QK^T MFMA steps along d
    static constexpr int EB = D / 32;            // 32-wide blocks of the output dim
    static constexpr int KCH = D / 8;            // 16-byte chunks per K or V row
    static constexpr int NQK = 2 * KK;           // MFMAs of one S tile
    static constexpr int NPV = 4 * EB;           // MFMAs of one PV tile
    // K rows padded by one 16-byte unit: the 16 lanes one LDS cycle serves
    // (rows r..r+15, same chunk) start 17 units apart, i.e. on 16 distinct
    // 4-bank groups of the 64 banks, with affine addresses.
    static constexpr int K_UNITS = KCH + 1;
    static constexpr int K_ROW_BYTES = 16 * K_UNITS;
    static constexpr int K_BYTES = kBN * K_ROW_BYTES;
    // V rows stay row-major (keys x dims) and are read transposed; rows are
    // padded to 80 dwords (D=128) / 48 dwords (D=64) so that the 4 rows x 2
    // column blocks one 32-lane transposed read touches map to all 64 banks.
    static constexpr int V_UNITS = KCH + 4;
    static constexpr int V_ROW_BYTES = 16 * V_UNITS;
    static constexpr int V_BYTES = kBN * V_ROW_BYTES;
    static constexpr int LDS_BYTES = 2 * K_BYTES + 2 * V_BYTES;   // K0 K1 V0 V1
    // Direct global->LDS loads: one wave instruction fills 64 consecutive
    // 16-byte units, so a tile takes K_UNITS (V_UNITS) instructions, dealt
    // round-robin to the wavefronts.
    static constexpr int K_DMA = K_UNITS;
    static constexpr int V_DMA = V_UNITS;
    static constexpr int K_DMA_PER_WAVE = (K_DMA + kWaves - 1) / kWaves;
    static constexpr int V_DMA_PER_WAVE = (V_DMA + kWaves - 1) / kWaves;
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

// Wait until this wavefront's direct global->LDS loads have landed
// (vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Lanes l and l+32 hold the two halves of one query row's keys: combine them
// with one v_permlane32_swap (each lane ends with {own, partner} in some order).
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(KParams p) {
    using TL = Tile<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // ---- decode the work unit -------------------------------------------
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
    const int64_t head_off = tok0 * ld + int64_t(head) * D;
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

    // ---- direct-load offsets and LDS read addresses -----------------------
    // DMA instruction n of a tile covers units [64n, 64n+64); lane i fetches
    // unit 64n+i = (row, chunk) of the padded LDS image.  Pad units fetch a
    // duplicate of the row's last chunk (never read back).
    uint32_t k_dma_off[TL::K_DMA_PER_WAVE], v_dma_off[TL::V_DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < TL::K_DMA_PER_WAVE; ++j) {
        const int u = 64 * (wave + kWaves * j) + lane;
        const int c = u % TL::K_UNITS;
        k_dma_off[j] = uint32_t(u / TL::K_UNITS) * row_bytes + 16u * uint32_t(c < TL::KCH ? c : TL::KCH - 1);
    }
#pragma unroll
    for (int j = 0; j < TL::V_DMA_PER_WAVE; ++j) {
        const int u = 64 * (wave + kWaves * j) + lane;
        const int c = u % TL::V_UNITS;
        v_dma_off[j] = uint32_t(u / TL::V_UNITS) * row_bytes + 16u * uint32_t(c < TL::KCH ? c : TL::KCH - 1);
    }
    // K fragment of lane: row l32 (+32 per key block), bytes 16*hlf (+32 per kk).
    const int k_rd = l32 * TL::K_ROW_BYTES + hlf * 16;
    // V^T fragment via two transposed reads: in each 16-lane group lane j
    // addresses row (4h + j/4) of the 16-key chunk (+8 rows for the second
    // read) at dims 32m + 16*(group&1) + 4*(j&3); lane i then receives dim
    // 32m + (lane&31) for 4 consecutive keys.
    const int v_rd = (4 * hlf + ((lane & 15) >> 2)) * TL::V_ROW_BYTES +
                     2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    auto kbuf = [&](int b) { return smem + b * TL::K_BYTES; };
    auto vbuf = [&](int b) { return smem + 2 * TL::K_BYTES + b * TL::V_BYTES; };

    // Direct loads of K/V tile `tile` into an LDS buffer (rows past the end
    // of the sequence read as zeros through the buffer range check).
    auto dma_k = [&](int tile, unsigned char* kb) {
        const uint32_t base = uint32_t(tile) * kBN * row_bytes;
#pragma unroll
        for (int j = 0; j < TL::K_DMA_PER_WAVE; ++j) {
            const int nidx = wave + kWaves * j;
            if (TL::K_DMA % kWaves == 0 || nidx < TL::K_DMA)
                dma16(k_rs, kb + 1024 * nidx, k_dma_off[j], base);
        }
    };
    auto dma_v = [&](int tile, unsigned char* vb) {
        const uint32_t base = uint32_t(tile) * kBN * row_bytes;
#pragma unroll
        for (int j = 0; j < TL::V_DMA_PER_WAVE; ++j) {
            const int nidx = wave + kWaves * j;
            if (TL::V_DMA % kWaves == 0 || nidx < TL::V_DMA)
                dma16(v_rs, vb + 1024 * nidx, v_dma_off[j], base);
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
    const bool ragged = (L % kBN) != 0;

    // Operand fragment of MFMA op `i`: S ops read K fragment i (key block
    // i&1, d-step i>>1); PV ops read the V^T fragment of (chunk i/EB, output
    // block i%EB) with two transposed reads (keys 4h..4h+3, 8+4h..8+4h+3).
    auto kfrag = [&](int i, const unsigned char* kb) -> bf16x8_t {
        return *reinterpret_cast<const bf16x8_t*>(kb + k_rd + (i & 1) * 32 * TL::K_ROW_BYTES + (i >> 1) * 32);
    };
    auto vfrag = [&](int j, const unsigned char* vb) -> bf16x8_t {
        const unsigned char* a = vb + v_rd + (j / TL::EB) * 16 * TL::V_ROW_BYTES + (j % TL::EB) * 64;
        const s16x4_t lo = lds_read_tr16_b64(a);
        const s16x4_t hi = lds_read_tr16_b64(a + 8 * TL::V_ROW_BYTES);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // One K/V tile t in buffers `cur`: S^T = K Q^T, online softmax,
    // O^T += V^T P^T.  The direct loads of tile t+1 into the other buffers
    // are issued first and land during this tile's work.
    auto step = [&](int t, const int cur, bool masked) {
        const unsigned char* kb = kbuf(cur);
        const unsigned char* vb = vbuf(cur);
        if (t + 1 < nkv) {
            dma_k(t + 1, kbuf(cur ^ 1));
            dma_v(t + 1, vbuf(cur ^ 1));
        }

        // S^T for the 64 keys: two 32-key accumulators; fragments read from
        // LDS kPrefetch MFMAs ahead (sched_barrier keeps them ahead).
        f32x16_t s[2];
        {
            bf16x8_t fr[kPrefetch];
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) fr[i] = kfrag(i, kb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TL::NQK; ++i) {
                const bf16x8_t f = fr[i % kPrefetch];
                if (i < 2)
                    s[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[0], f32x16_t{}, 0, 0, 0);
                else
                    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[i >> 1], s[i & 1], 0, 0, 0);
                if (i + kPrefetch < TL::NQK) fr[i % kPrefetch] = kfrag(i + kPrefetch, kb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (masked) {
            const int kv0 = t * kBN;
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
        mx = half_max(mx) * c;
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
        bf16x8_t pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int bb = cc >> 1, r0 = 8 * (cc & 1);
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r0 + i], c, -m_run));
                lsum += e[i];
            }
            u32x4_t u;
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
            pf[cc] = __builtin_bit_cast(bf16x8_t, u);
        }
        l_run += lsum;

        // O^T += V^T P^T over EB independent accumulators, chunk outer.
        {
            bf16x8_t fr[kPrefetch];
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) fr[i] = vfrag(i, vb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TL::NPV; ++i) {
                const bf16x8_t f = fr[i % kPrefetch];
                oacc[i % TL::EB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[i / TL::EB],
                                                                          oacc[i % TL::EB], 0, 0, 0);
                if (i + kPrefetch < TL::NPV) fr[i % kPrefetch] = vfrag(i + kPrefetch, vb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_dma();
        __syncthreads();
    };

    dma_k(0, kbuf(0));
    dma_v(0, vbuf(0));
    wait_dma();
    __syncthreads();
    const int nfull = ragged ? nkv - 1 : nkv;
    int t = 0;
    for (; t + 2 <= nfull; t += 2) {       // unrolled pair: buffers 0 then 1
        step(t, 0, false);
        step(t + 1, 1, false);
    }
    if (t < nfull) {
        step(t, 0, false);
        ++t;
    }
    if (t < nkv) step(t, t & 1, true);

    // ---- epilogue -------------------------------------------------------
    const float l_tot = half_sum(l_run);
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
    const size_t smem = Tile<D>::LDS_BYTES;
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
