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
//  * Work = (sequence, head, 256-query tile, 64-key step).  Sequences are
//    ordered longest first (in-kernel for packs of up to 64 sequences,
//    otherwise by a one-workgroup prologue kernel writing into the caller's
//    workspace); within a sequence the order is head-major, then q-tile.
//  * Stream-K: a persistent grid of one workgroup per CU; workgroup g takes
//    the contiguous range [g*W/G, (g+1)*W/G) of the W (tile, key-step)
//    iterations, so mixed lengths and tile counts that are not a multiple of
//    the CU count leave no CU idle.  A tile cut by a range boundary leaves
//    partial results (unnormalised O in bf16, reference max and sum in fp32)
//    in the workspace; a fix-up kernel merges them with the log-sum-exp rule.
//    The partition is fixed by (W, G), so results are deterministic.
//    Logical workgroups map to blockIdx so that consecutive ranges (same
//    sequence and head, hence the same K/V) run on one XCD and share its L2.
//  * 8 wavefronts (2 per SIMD, <= 256 VGPRs each) share every K/V tile; each
//    wavefront owns 32 query rows, held in VGPRs as MFMA B operands.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: every lane holds 16 keys of one query row, so
//    the online-softmax max/sum need one v_permlane32_swap and the rescale of
//    the output accumulator is a per-lane scalar.  The fp32 probabilities are
//    rounded to bf16 in registers and used directly as the B operand of
//    O^T += V^T P^T: the S^T accumulator layout gives each lane keys
//    {4h..4h+3, 8+4h..8+4h+3} of every 16-key chunk, which is exactly what
//    two transposed LDS reads (ds_read_b64_tr_b16) of the row-major V tile
//    deliver as the V^T operand.
//  * Per 64-key tile a wavefront runs S^T = K Q^T (2*D/16 MFMAs), the online
//    softmax (VALU), then O^T += V^T P^T (D/8 MFMAs).  The two wavefronts of
//    a SIMD are half a tile apart: waves 0..3 run S, softmax, PV of tile i
//    between two barriers while waves 4..7 run softmax, PV of tile i and S
//    of tile i+1, so one wave's softmax overlaps the other's MFMAs.  Operand
//    fragments are read from LDS four MFMAs ahead, pinned with
//    sched_barrier so the scheduler does not sink them next to their use.
//  * K and V arrive by direct global->LDS buffer loads (no staging
//    registers, no LDS stores) issued by waves 0..3, two K tiles and one V
//    tile ahead of use (3 K buffers, 2 V buffers), one barrier per tile.
//    Rows are padded (K: 2D -> 2D+16 bytes, V: 2D -> 2D+64) so every LDS
//    read cycle hits distinct banks of the 64, with affine addresses.
//  * Q/K/V are read through raw buffer resources that end at the sequence's
//    last row, so ragged tiles read zeros without branches; only the last
//    key tile of a sequence masks its scores.
//  * exp2 with the softmax scale folded into one FMA (scale * log2 e); the
//    reference max is raised lazily (only when a row max grows by more than
//    2^8), so the output accumulator is rarely rescaled; all softmax state
//    in fp32.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kWaves = 8;        // wavefronts per workgroup: 2 per SIMD
constexpr int kBM = 32 * kWaves; // query rows per tile (32 per wavefront)
constexpr int kBN = 64;          // keys per K/V step
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;         // XCDs of an MI355X; blockIdx round-robins over them
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kInlineSeqs = 64;  // packs up to this many sequences schedule in-kernel
constexpr int kPrefetch = 4;     // MFMA operand fragments read ahead from LDS
constexpr int kLoaders = kWaves / 2;  // leading wavefronts, which issue the K/V loads

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
    static constexpr int K_STAGES = 3;           // K of tiles i, i+1, i+2
    static constexpr int V_STAGES = 2;           // V of tiles i, i+1
    static constexpr int LDS_BYTES = K_STAGES * K_BYTES + V_STAGES * V_BYTES;
    // Direct global->LDS loads: one wave instruction fills 64 consecutive
    // 16-byte units, so a tile takes K_UNITS (V_UNITS) instructions, dealt
    // round-robin to the leading wavefronts.
    static constexpr int K_DMA = K_UNITS;
    static constexpr int V_DMA = V_UNITS;
    static constexpr int K_DMA_PER_WAVE = (K_DMA + kLoaders - 1) / kLoaders;
    static constexpr int V_DMA_PER_WAVE = (V_DMA + kLoaders - 1) / kLoaders;
    // One partial-result slot of the workspace: unnormalised O (rounded to
    // bf16, kBM x D), then the reference max (log2 units) and sum of each
    // row in fp32.
    static constexpr size_t SLOT_BYTES = size_t(kBM) * D * 2 + size_t(kBM) * 8;
};

// ---------------------------------------------------------------------------
// Schedule.  Per rank r (sequences sorted longest first, ties by index):
// seq[r], tiles[r] = ceil(L/kBM), nkv[r] = ceil(L/kBN) and the exclusive
// prefix it_start[r] of tiles*H*nkv (it_start[n] = W, the total number of
// (tile, key-step) iterations).  Workspace header (bytes): [0,8) W,
// [8,12) n, then int32 seq[n], tiles[n], nkv[n], then (8-aligned) int64
// it_start[n+1]; partial slots start at the next 256-byte boundary.
// ---------------------------------------------------------------------------
struct Sched {
    const int32_t* seq;
    const int32_t* tiles;
    const int32_t* nkv;
    const int64_t* it_start;
    int n;
    int64_t W;
};

__host__ __device__ constexpr size_t sched_ints_end(int n) { return size_t(12) + size_t(12) * n; }
__host__ __device__ constexpr size_t sched_prefix_off(int n) { return (sched_ints_end(n) + 7) / 8 * 8; }
__host__ __device__ constexpr size_t sched_bytes(int n) {
    return (sched_prefix_off(n) + size_t(8) * (n + 1) + 255) / 256 * 256;
}

// Build the schedule into the given arrays (LDS or global); every thread of
// the block calls it.
__device__ void build_schedule(const int32_t* __restrict__ cu, int n, int H, int32_t* seq,
                               int32_t* tiles, int32_t* nkv, int64_t* it_start) {
    for (int s = threadIdx.x; s < n; s += blockDim.x) {
        const int Ls = cu[s + 1] - cu[s];
        int rank = 0;
        for (int i = 0; i < n; ++i) {
            const int Li = cu[i + 1] - cu[i];
            rank += (Li > Ls) || (Li == Ls && i < s);
        }
        seq[rank] = s;
        tiles[rank] = (Ls + kBM - 1) / kBM;
        nkv[rank] = (Ls + kBN - 1) / kBN;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t acc = 0;
        for (int r = 0; r < n; ++r) {
            it_start[r] = acc;
            acc += int64_t(tiles[r]) * H * nkv[r];
        }
        it_start[n] = acc;
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void attn_schedule_kernel(const int32_t* __restrict__ cu, int n,
                                                            int H, unsigned char* __restrict__ ws) {
    int32_t* ints = reinterpret_cast<int32_t*>(ws + 8);
    int64_t* pre = reinterpret_cast<int64_t*>(ws + sched_prefix_off(n));
    build_schedule(cu, n, H, ints + 1, ints + 1 + n, ints + 1 + 2 * n, pre);
    if (threadIdx.x == 0) {
        *reinterpret_cast<int64_t*>(ws) = pre[n];
        ints[0] = n;
    }
}

// Schedule of this call: built in LDS for small packs, else the prologue's.
struct SchedLds {
    int32_t seq[kInlineSeqs], tiles[kInlineSeqs], nkv[kInlineSeqs];
    int64_t it_start[kInlineSeqs + 1];
};

__device__ Sched get_schedule(const int32_t* cu, int n, int H, const unsigned char* ws, SchedLds& lds) {
    Sched s;
    s.n = n;
    if (n <= kInlineSeqs) {
        build_schedule(cu, n, H, lds.seq, lds.tiles, lds.nkv, lds.it_start);
        s.seq = lds.seq;
        s.tiles = lds.tiles;
        s.nkv = lds.nkv;
        s.it_start = lds.it_start;
    } else {
        const int32_t* ints = reinterpret_cast<const int32_t*>(ws + 8);
        s.seq = ints + 1;
        s.tiles = ints + 1 + n;
        s.nkv = ints + 1 + 2 * n;
        s.it_start = reinterpret_cast<const int64_t*>(ws + sched_prefix_off(n));
    }
    s.W = s.it_start[n];
    return s;
}

// First iteration of logical workgroup g of G.
__device__ __forceinline__ int64_t range_begin(int64_t W, int g, int G) { return W * g / G; }

// Logical workgroup of this block: consecutive logical ranges share an XCD
// (blockIdx round-robins over the XCDs).
__device__ __forceinline__ int logical_wg(int b, int G) {
    if (G % kXcds != 0) return b;
    return (b % kXcds) * (G / kXcds) + b / kXcds;
}

// The tile containing iteration `it`: rank, tile index within the rank and
// key step within the tile.
struct TileAt {
    int rank, tile, step;
};
__device__ __forceinline__ TileAt locate(const Sched& s, int64_t it) {
    int lo = 0, hi = s.n - 1;            // last rank with it_start <= it
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.it_start[mid] <= it) lo = mid; else hi = mid - 1;
    }
    const int64_t local = it - s.it_start[lo];
    const int nk = s.nkv[lo];
    TileAt t;
    t.rank = lo;
    t.tile = int(local / nk);
    t.step = int(local - int64_t(t.tile) * nk);
    return t;
}

struct KParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* cu;
    unsigned char* ws;
    int n_seq;
    int G;               // persistent workgroups (= CUs)
    int64_t T;
    int64_t ld_qkv, ld_o;
    int H;
    float scale_log2;    // softmax_scale * log2(e)
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
    __shared__ SchedLds sched_lds;

    const Sched sch = get_schedule(p.cu, p.n_seq, p.H, p.ws, sched_lds);
    const int g = logical_wg(blockIdx.x, p.G);
    const int64_t it_end = range_begin(sch.W, g + 1, p.G);
    unsigned char* const partials = p.ws + sched_bytes(p.n_seq);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    // Waves 0..3 (one per SIMD) lead and issue the direct loads; waves 4..7
    // trail them by one softmax phase (see the step loop below).
    const bool lead = wave < kLoaders;
    const int lw = wave & (kLoaders - 1);
    const int64_t ld = p.ld_qkv;
    const uint32_t row_bytes = uint32_t(ld) * 2u;
    const float c = p.scale_log2;

    // ---- direct-load offsets and LDS read addresses (same for every tile) --
    // DMA instruction n of a tile covers units [64n, 64n+64); lane i fetches
    // unit 64n+i = (row, chunk) of the padded LDS image.  Pad units fetch a
    // duplicate of the row's last chunk (never read back).  Instruction n is
    // issued by leading wave n % kLoaders.
    uint32_t k_dma_off[TL::K_DMA_PER_WAVE], v_dma_off[TL::V_DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < TL::K_DMA_PER_WAVE; ++j) {
        const int u = 64 * (lw + kLoaders * j) + lane;
        const int cc = u % TL::K_UNITS;
        k_dma_off[j] = uint32_t(u / TL::K_UNITS) * row_bytes + 16u * uint32_t(cc < TL::KCH ? cc : TL::KCH - 1);
    }
#pragma unroll
    for (int j = 0; j < TL::V_DMA_PER_WAVE; ++j) {
        const int u = 64 * (lw + kLoaders * j) + lane;
        const int cc = u % TL::V_UNITS;
        v_dma_off[j] = uint32_t(u / TL::V_UNITS) * row_bytes + 16u * uint32_t(cc < TL::KCH ? cc : TL::KCH - 1);
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
    auto vbuf = [&](int b) { return smem + TL::K_STAGES * TL::K_BYTES + b * TL::V_BYTES; };

    bool first_segment = true;
    for (int64_t it = range_begin(sch.W, g, p.G); it < it_end;) {
        // ---- the segment: one tile's key steps [kv0, kv1) -------------------
        // The segment is the same for every lane; readfirstlane says so, so
        // that the buffer resources and offsets below live in SGPRs.
        const TileAt at = locate(sch, it);
        const int rank = __builtin_amdgcn_readfirstlane(at.rank);
        const int seq = __builtin_amdgcn_readfirstlane(sch.seq[rank]);
        const int nt = __builtin_amdgcn_readfirstlane(sch.tiles[rank]);
        const int nkv = __builtin_amdgcn_readfirstlane(sch.nkv[rank]);
        const int tile = __builtin_amdgcn_readfirstlane(at.tile);
        const int kv0 = __builtin_amdgcn_readfirstlane(at.step);
        const int kv1 = __builtin_amdgcn_readfirstlane(int(min(int64_t(nkv), int64_t(kv0) + (it_end - it))));
        const int head = tile / nt;
        const int qtile = tile - head * nt;
        const int64_t tok0 = __builtin_amdgcn_readfirstlane(p.cu[seq]);
        const int L = __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);
        // the last key tile of a sequence whose length is not a multiple of
        // kBN has keys past the end: those scores are masked
        const int masked_tile = (L % kBN) != 0 ? nkv - 1 : nkv;
        it += kv1 - kv0;

        // Buffer resources over this sequence's rows of the head: loads of
        // rows at or past L return zeros (ragged q-tile and last key tile).
        const uint64_t seq_bytes = uint64_t(L) * uint64_t(ld) * 2u;
        const int64_t head_off = tok0 * ld + int64_t(head) * D;
        const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + head_off, seq_bytes);
        const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + head_off, seq_bytes);
        const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + head_off, seq_bytes);

        // Direct loads of key tile `t` into K buffer kb / V buffer vb
        // (leading waves only).
        auto dma_k = [&](int t, int kb) {
            const uint32_t base = uint32_t(t) * kBN * row_bytes;
#pragma unroll
            for (int j = 0; j < TL::K_DMA_PER_WAVE; ++j) {
                const int nidx = lw + kLoaders * j;
                if (TL::K_DMA % kLoaders == 0 || nidx < TL::K_DMA)
                    dma16(k_rs, kbuf(kb) + 1024 * nidx, k_dma_off[j], base);
            }
        };
        auto dma_v = [&](int t, int vb) {
            const uint32_t base = uint32_t(t) * kBN * row_bytes;
#pragma unroll
            for (int j = 0; j < TL::V_DMA_PER_WAVE; ++j) {
                const int nidx = lw + kLoaders * j;
                if (TL::V_DMA % kLoaders == 0 || nidx < TL::V_DMA)
                    dma16(v_rs, vbuf(vb) + 1024 * nidx, v_dma_off[j], base);
            }
        };
        auto dma = [&](int t, int kb, int vb) {
            dma_k(t, kb);
            dma_v(t, vb);
        };

        // Q^T fragments (B operand), kept in registers.
        const int qrow = qtile * kBM + wave * 32 + l32;    // row inside the sequence
        bf16x8_t qf[TL::KK];
        {
            const uint32_t qoff = uint32_t(qrow) * row_bytes + 16u * hlf;
#pragma unroll
            for (int kk = 0; kk < TL::KK; ++kk)
                qf[kk] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, qoff, 32u * kk));
        }

        f32x16_t oacc[TL::EB];
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
        float m_run = -INFINITY;
        float l_run = 0.f;

        // Operand fragments: S op i reads K fragment i (key block i&1, d-step
        // i>>1); PV op j reads the V^T fragment of (chunk j/EB, output block
        // j%EB) with two transposed reads (keys 4h..4h+3, 8+4h..8+4h+3).
        auto kfrag = [&](int i, const unsigned char* kb) -> bf16x8_t {
            return *reinterpret_cast<const bf16x8_t*>(kb + k_rd + (i & 1) * 32 * TL::K_ROW_BYTES + (i >> 1) * 32);
        };
        auto vfrag = [&](int j, const unsigned char* vb) -> bf16x8_t {
            const unsigned char* a = vb + v_rd + (j / TL::EB) * 16 * TL::V_ROW_BYTES + (j % TL::EB) * 64;
            const s16x4_t lo = lds_read_tr16_b64(a);
            const s16x4_t hi = lds_read_tr16_b64(a + 8 * TL::V_ROW_BYTES);
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };

        // S^T = K Q^T for one key tile held in K buffer kb.
        f32x16_t s[2];
        auto qk = [&](const unsigned char* __restrict__ kb) {
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
        };

        // Online softmax of key tile t (scores in s) for this lane's query
        // row, then O^T += V^T P^T with the tile's V in buffer vb.  The
        // exponentials use a reference max m_run that is only raised when a
        // row's block max exceeds it by more than kRescaleLog2 (so p <=
        // 2^kRescaleLog2); numerator and denominator share m_run, so the
        // result is the same softmax, and the output accumulator is rescaled
        // only on those (rare, wave-uniform) occasions.
        auto softmax_pv = [&](int t, const unsigned char* __restrict__ vb) {
            if (t == masked_tile) {
                const int key0 = t * kBN;
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * bb + 8 * (r >> 2) + 4 * hlf + (r & 3);
                        if (key >= L) s[bb][r] = -INFINITY;
                    }
            }
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
        };

        // ---- key steps -----------------------------------------------------
        // Iteration i (0 <= i <= n) runs softmax + PV of tile i-1, then S of
        // tile i; the leading waves pass the step barrier between the two,
        // the trailing waves after both.  Between two barriers a leading wave
        // thus runs S(i), softmax(i), PV(i) while a trailing wave runs
        // softmax(i), PV(i), S(i+1): on each SIMD one wave's softmax (VALU)
        // overlaps the other wave's MFMAs instead of both alternating in
        // lockstep.  In that interval K of tiles i and i+1 and V of tile i
        // are read, so K of tile i+2 and V of tile i+1 are fetched into the
        // third K buffer and the second V buffer (K of tile i in buffer i%3,
        // V in buffer i%2).  Only the leading waves load; each barrier
        // follows its wave's own loads landing.
        const int n = kv1 - kv0;
        if (lead) {
            dma(kv0, 0, 0);
            if (n > 1) dma_k(kv0 + 1, 1);
        }
        wait_dma();
        __syncthreads();
        int k0 = 0, k1 = 1, k2 = 2, v0 = 0;     // K buffers of tiles i, i+1, i+2; V of tile i
        for (int i = 0; i <= n; ++i) {
            if (i > 0) softmax_pv(kv0 + i - 1, vbuf(v0 ^ 1));
            if (lead) {
                wait_dma();
                __syncthreads();
                if (i + 2 < n) dma_k(kv0 + i + 2, k2);
                if (i + 1 < n) dma_v(kv0 + i + 1, v0 ^ 1);
            }
            if (i < n) qk(kbuf(k0));
            if (!lead) {
                wait_dma();
                __syncthreads();
            }
            const int kt = k0;
            k0 = k1;
            k1 = k2;
            k2 = kt;
            v0 ^= 1;
        }

        // ---- epilogue ----------------------------------------------------
        const float l_tot = half_sum(l_run);
        if (kv0 == 0 && kv1 == nkv) {
            // whole tile: normalise and store O (bf16) and the LSE
            if (qrow < L) {
                const float inv = 1.0f / l_tot;
                uint16_t* op = p.o + (tok0 + qrow) * p.ld_o + int64_t(head) * D + 4 * hlf;
#pragma unroll
                for (int m = 0; m < TL::EB; ++m)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        u32x2_t val;
                        val[0] = pack_bf16x2(oacc[m][4 * gq] * inv, oacc[m][4 * gq + 1] * inv);
                        val[1] = pack_bf16x2(oacc[m][4 * gq + 2] * inv, oacc[m][4 * gq + 3] * inv);
                        *reinterpret_cast<u32x2_t*>(op + 32 * m + 8 * gq) = val;
                    }
                if (p.lse != nullptr && hlf == 0)
                    p.lse[int64_t(head) * p.T + tok0 + qrow] = m_run * 0.69314718055994531f + logf(l_tot);
            }
        } else {
            // piece of a tile shared with other workgroups: partial in slot
            // 2g (this workgroup's first segment) or 2g+1 (its last)
            unsigned char* slot = partials + size_t(2 * g + (first_segment ? 0 : 1)) * TL::SLOT_BYTES;
            uint16_t* acc = reinterpret_cast<uint16_t*>(slot);
            float* ml = reinterpret_cast<float*>(slot + size_t(kBM) * D * 2);
            const int row = wave * 32 + l32;
#pragma unroll
            for (int m = 0; m < TL::EB; ++m)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2_t val;
                    val[0] = pack_bf16x2(oacc[m][4 * gq], oacc[m][4 * gq + 1]);
                    val[1] = pack_bf16x2(oacc[m][4 * gq + 2], oacc[m][4 * gq + 3]);
                    *reinterpret_cast<u32x2_t*>(acc + row * D + 32 * m + 8 * gq + 4 * hlf) = val;
                }
            if (hlf == 0) {
                ml[row] = m_run;
                ml[kBM + row] = l_tot;
            }
        }
        first_segment = false;
    }
}

// Merge the partial pieces of every tile that a range boundary cut.  Block
// b-1 handles boundary b (1 <= b < G) if b is the first boundary inside its
// tile; the pieces come from workgroup b-1 (slot 2(b-1), or 2(b-1)+1 if the
// tile is not its first segment) and from every non-empty workgroup g >= b
// whose range starts inside the tile (slot 2g).
//   O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,  LSE = M ln 2 + ln(sum)
constexpr int kFixThreads = 1024;   // 4 threads per query row of a tile

template <int D>
__global__ __launch_bounds__(kFixThreads) void attn_fixup_kernel(KParams p) {
    using TL = Tile<D>;
    __shared__ SchedLds sched_lds;
    __shared__ int slots[1024];
    __shared__ int n_slots;
    const Sched sch = get_schedule(p.cu, p.n_seq, p.H, p.ws, sched_lds);
    const int G = p.G;
    const int b = blockIdx.x + 1;
    const int64_t Bb = range_begin(sch.W, b, G);
    if (Bb >= sch.W) return;
    const TileAt at = locate(sch, Bb);
    if (at.step == 0) return;                                // boundary on a tile start
    const int64_t tile_start = Bb - at.step;
    if (range_begin(sch.W, b - 1, G) > tile_start) return;   // an earlier boundary handles it
    const int nkv = sch.nkv[at.rank];
    const int64_t tile_end = tile_start + nkv;

    if (threadIdx.x == 0) {
        int ns = 0;
        const int g0 = b - 1;
        slots[ns++] = 2 * g0 + (range_begin(sch.W, g0, G) == tile_start ? 0 : 1);
        for (int gg = b; gg < G && range_begin(sch.W, gg, G) < tile_end && ns < 1024; ++gg)
            if (range_begin(sch.W, gg + 1, G) > range_begin(sch.W, gg, G)) slots[ns++] = 2 * gg;
        n_slots = ns;
    }
    __syncthreads();

    const int seq = sch.seq[at.rank];
    const int nt = sch.tiles[at.rank];
    const int head = at.tile / nt;
    const int qtile = at.tile - head * nt;
    const int64_t tok0 = p.cu[seq];
    const int L = p.cu[seq + 1] - int(tok0);
    const unsigned char* partials = p.ws + sched_bytes(p.n_seq);
    const int ns = n_slots;
    auto slot_at = [&](int i) { return partials + size_t(slots[i]) * TL::SLOT_BYTES; };
    auto ml_at = [&](int i) { return reinterpret_cast<const float*>(slot_at(i) + size_t(kBM) * D * 2); };

    // per row: the reference max M over the pieces and 1 / total weight
    __shared__ float row_m[kBM], row_inv[kBM];
    const int tid = threadIdx.x;
    if (tid < kBM) {
        float M = -INFINITY;
        for (int i = 0; i < ns; ++i) M = fmaxf(M, ml_at(i)[tid]);
        float lt = 0.f;
        for (int i = 0; i < ns; ++i) lt += exp2f(ml_at(i)[tid] - M) * ml_at(i)[kBM + tid];
        row_m[tid] = M;
        row_inv[tid] = 1.0f / lt;
        const int qrow = qtile * kBM + tid;
        if (p.lse != nullptr && qrow < L) p.lse[int64_t(head) * p.T + tok0 + qrow] = M * 0.69314718055994531f + logf(lt);
    }
    __syncthreads();

    // weighted sum of the pieces over the tile's 16-byte chunks (8 bf16) in
    // memory order (consecutive lanes read consecutive chunks)
    constexpr int kRowChunks = D / 8;
    constexpr int kChunks = kBM * kRowChunks;
    static_assert(kChunks % kFixThreads == 0, "whole chunks per thread");
#pragma unroll
    for (int j = 0; j < kChunks / kFixThreads; ++j) {
        const int cidx = tid + kFixThreads * j;
        const int row = cidx / kRowChunks;
        const int qrow = qtile * kBM + row;
        if (qrow >= L) continue;
        const float M = row_m[row];
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < ns; ++i) {
            const float w = exp2f(ml_at(i)[row] - M);
            float a8[8];
            unpack8(reinterpret_cast<const u32x4_t*>(slot_at(i))[cidx], a8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += w * a8[e];
        }
        const float inv = row_inv[row];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
        st16(p.o + (tok0 + qrow) * p.ld_o + int64_t(head) * D + 8 * (cidx % kRowChunks), pack8(acc));
    }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
    const int G = device_cu_count();
    if (G <= 0) return hipErrorInvalidDevice;
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    if (a.n_seq > kInlineSeqs) {
        hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seq, a.H, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    KParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
    p.cu = a.cu_seqlens; p.ws = ws; p.n_seq = a.n_seq; p.G = G; p.T = a.T;
    p.ld_qkv = a.ld_qkv; p.ld_o = a.ld_o; p.H = a.H;
    p.scale_log2 = a.softmax_scale * 1.4426950408889634f;
    const size_t smem = Tile<D>::LDS_BYTES;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_fwd_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(smem));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(G), dim3(kThreads), smem, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (G > 1) {
        hipLaunchKernelGGL(attn_fixup_kernel<D>, dim3(G - 1), dim3(kFixThreads), 0, stream, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

size_t attn_workspace_bytes(int32_t n_seq, int64_t /*T*/, int32_t /*H*/, int32_t D) {
    const int n = n_seq < 0 ? 0 : n_seq;
    int G = device_cu_count();
    if (G <= 0) G = 256;   // no device visible: size for an MI355X
    const size_t slot = D == 64 ? Tile<64>::SLOT_BYTES : Tile<128>::SLOT_BYTES;
    return sched_bytes(n) + size_t(2) * G * slot;
}

hipError_t launch_varlen_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_d<128>(a, stream);
    return launch_d<64>(a, stream);
}

}  // namespace mf
