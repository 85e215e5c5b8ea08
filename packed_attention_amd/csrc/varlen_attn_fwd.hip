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
//  * Work = (sequence, head, 256-query tile, 32-key step).  Sequences are
//    ordered by descending octave of their key-step count, ties by index
//    (in-kernel for packs of up to 64 sequences, otherwise by a one-workgroup
//    O(n) prologue kernel writing into the caller's workspace); within a
//    sequence the order is head-major, then q-tile.
//  * Stream-K: a persistent grid of one workgroup per CU; workgroup g takes
//    the contiguous range [g*W/G, (g+1)*W/G) of the W (tile, key-step)
//    iterations, so mixed lengths and tile counts that are not a multiple of
//    the CU count leave no CU idle.  A tile cut by a range boundary leaves
//    partial results (unnormalised O, reference max and sum, all in fp32)
//    in the workspace; a fix-up kernel merges them with the log-sum-exp rule.
//    The partition is fixed by (W, G), so results are deterministic.
//    Logical workgroups map to blockIdx so that consecutive ranges (same
//    sequence and head, hence the same K/V) run on one XCD and share its L2.
//  * A workgroup owns a 256-row query tile and runs four wavefronts, one
//    per SIMD, each owning 64 query rows as two 32-row blocks, so that each
//    K or V fragment read from LDS feeds two MFMAs.  (Eight wavefronts of 32
//    rows, two per SIMD, were faster on isolated calls but slower on calls
//    back to back, where the clock settles lower: the four-wavefront form
//    reads half the LDS bytes per MFMA.)  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: every lane holds 16 keys of
//    one query row, so a row's statistics combine lanes l and l+32 with one
//    v_permlane32_swap.  The fp32 probabilities are rounded to bf16 in
//    registers and used directly as the B operand of O^T += V^T P^T: the S^T
//    accumulator layout gives each lane keys {4h..4h+3, 8+4h..8+4h+3} of
//    every 16-key chunk, which is exactly what two transposed LDS reads
//    (ds_read_b64_tr_b16) of the row-major V tile deliver as the V^T operand.
//  * Per step t a wavefront runs two phases, with the softmax VALU work
//    threaded between the MFMAs of the same wavefront:
//      phase 1: S(t+1) = K(t+1) Q^T   ||  p = exp2(x(t)) in place, bf16 rounding
//      phase 2: O += V(t)^T P(t)^T     ||  row sums of p(t), x(t+1) = S(t+1) * scale*log2e - m
//    Operand fragments are read from LDS three MFMAs ahead.  The step carries
//    no other VALU work: the reference max m of each row is fixed by the
//    segment's first key step (numerator and denominator share it, so the
//    softmax is unchanged), and a row sum above 2^64 at the segment's end --
//    the only way a probability can have overflowed -- makes the workgroup
//    redo the segment with exact row maxima from a scores-only pass.
//  * K and V arrive by direct global->LDS buffer loads (no staging registers,
//    no LDS stores), issued by every wavefront from inline assembly (the
//    compiler would otherwise order every transposed LDS read behind all
//    outstanding direct loads); completion is tracked with explicit vmcnt
//    waits.  K and V each have a ring of 8 stages of 32 rows: during step t,
//    K of tiles t+1..t+7 and V of tiles t..t+6 are resident and K(t+8) and
//    V(t+7) are loading, so a load has five steps to land, and one barrier
//    per step publishes them.  The step loop runs in groups of 8 steps with
//    the ring positions known at compile time, so every LDS stage address
//    is an immediate offset from per-lane base registers and the loop
//    carries almost no address arithmetic; the steps that do not fill a
//    group run first.  Every step issues the same number of loads (a tile
//    past the segment is addressed out of range, which returns zeros
//    without memory traffic), so the wait count is a constant.  LDS rows are
//    not padded: the 16-byte units of each row are XOR-swizzled so that
//    every LDS read cycle of the K reads and of the transposed V reads
//    touches 64 distinct banks.
//  * Q/K/V are read through raw buffer resources that end at the sequence's
//    last row, so ragged tiles read zeros without branches.  A tile's key
//    steps take the sequence's last (ragged) key tile first, so only that
//    first step masks its scores and the step loop has no mask branch.
//  * exp2 with the softmax scale folded into one FMA (scale * log2 e); all
//    softmax state in fp32, row sums of the fp32 probabilities.
#include <atomic>
#include <cmath>
#include <mutex>
#include <utility>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kBM = 256;             // query rows per tile (one workgroup)
constexpr int kBN = 32;              // keys per K/V step (one 32-key MFMA block)
constexpr int kXcds = 8;             // XCDs of an MI355X; blockIdx round-robins over them
constexpr float kSumLimit = 1.8446744e19f;  // 2^64: bound on a row sum before the exact-max redo
constexpr int kInlineSeqs = 64;      // packs up to this many sequences schedule in-kernel
// K and V stages in LDS: rings of kRing tiles (tile j lives in stage
// (j + phase offset) mod kRing).  During step t, K of tiles t+1 .. t+7 and V
// of tiles t .. t+6 are resident and the loads of K(t+8) and V(t+7) fill the
// stages freed by tiles t and t-1.
constexpr int kRing = 8;
constexpr int kKStages = kRing;
constexpr int kVStages = kRing;
constexpr int kSlack = kRing - 3;    // steps a direct load may stay in flight
static_assert((kRing & (kRing - 1)) == 0, "ring positions are taken mod kRing with a mask");
constexpr int kPfK = 3;              // K fragments read ahead of their MFMA
constexpr int kPfV = 3;              // V fragments read ahead of their MFMA
constexpr uint32_t kOutOfRange = 0x80000000u;  // scalar offset past any sequence's rows

template <int D>
struct Tile {
    // 32-row blocks per wavefront: each K or V fragment feeds NB MFMAs.
    static constexpr int NB = 2;
    static constexpr int ROWS_W = 32 * NB;         // query rows per wavefront
    static constexpr int WAVES = kBM / ROWS_W;     // wavefronts per workgroup
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KK = D / 16;              // QK^T MFMA steps along d
    static constexpr int EB = D / 32;              // 32-wide blocks of the output dim
    static constexpr int U = D / 8;                // 16-byte units per K or V row
    static constexpr int R = 16 / U;               // rows per 256-byte line of the 64 banks
    static constexpr int ROW_BYTES = 2 * D;        // K/V rows are stored unpadded
    static constexpr int TILE_BYTES = kBN * ROW_BYTES;
    static constexpr int NI = TILE_BYTES / 1024;   // direct-load instructions per tile
    static constexpr int NI_W = NI / WAVES;        // ... issued by each wavefront
    static constexpr int NS = KK * NB;             // S MFMAs per step (KK d-steps x NB row blocks)
    static constexpr int NP = 2 * EB * NB;         // PV MFMAs per step (2 chunks x EB x NB row blocks)
    static constexpr int NV_FR = 2 * EB;           // V fragments per step
    static constexpr int LDS_BYTES = (kKStages + kVStages) * TILE_BYTES;
    // One partial-result slot of the workspace: unnormalised O (fp32, kBM x
    // D, so a cut tile's O is rounded to bf16 once, as a whole tile's), then
    // the reference max (log2 units) and sum of each row in fp32.
    static constexpr size_t SLOT_BYTES = size_t(kBM) * D * 4 + size_t(kBM) * 8;
    static_assert(NI % WAVES == 0, "whole direct-load instructions per wavefront");
};

// XOR swizzles of the 16-byte units of LDS row `row` (unit u is stored at
// u ^ swz(row)).  K: the 16 rows that one ds_read_b128 cycle serves fall on
// 16 distinct units of the 64 banks.  V: the 4 rows x 4 units that 32 lanes
// of one transposed read touch fall on 16 distinct units.
template <int D>
__device__ __forceinline__ constexpr int swz_k(int row) {
    return (row / Tile<D>::R) % Tile<D>::U;
}
template <int D>
__device__ __forceinline__ constexpr int swz_v(int row) {
    return 4 * ((row / Tile<D>::R) % (Tile<D>::U / 4));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Schedule.  Per rank r: seq[r], tiles[r] = ceil(L/kBM), nkv[r] = ceil(L/kBN)
// and the exclusive prefix it_start[r] of tiles*H*nkv (it_start[n] = W, the
// total number of (tile, key-step) iterations).  Sequences are ranked by
// descending octave floor(log2(nkv)) of their key-step count, ties by
// sequence index (empty sequences last).  Workspace header (bytes): [0,8) W,
// [8,12) n, then int32 seq[n], tiles[n], nkv[n], then (8-aligned) int64
// it_start[n+1]; partial slots start at the next 256-byte boundary.
// ---------------------------------------------------------------------------
struct Sched {
    const int32_t* seq;
    const int32_t* tiles;
    const int32_t* nkv;
    const int64_t* it_start;
    const int32_t* tok0;   // first token and length of each rank's sequence
    const int32_t* len;    // (in-LDS schedules only; nullptr otherwise)
    int n;
    int64_t W;
};

constexpr int kOctaves = 32;   // octave classes of the key-step count (class 0: empty)

__host__ __device__ constexpr size_t sched_ints_end(int n) { return size_t(12) + size_t(12) * n; }
__host__ __device__ constexpr size_t sched_prefix_off(int n) { return (sched_ints_end(n) + 7) / 8 * 8; }
__host__ __device__ constexpr size_t sched_bytes(int n) {
    return (sched_prefix_off(n) + size_t(8) * (n + 1) + 255) / 256 * 256;
}

// Octave class of a sequence of L tokens: 1 + floor(log2(ceil(L / kBN))),
// 0 for an empty sequence.
__device__ __forceinline__ int octave_class(int L) {
    const int nk = (L + kBN - 1) / kBN;
    return nk == 0 ? 0 : 32 - __clz(nk);
}

// In-kernel schedule of a small pack (n <= kInlineSeqs), built in LDS by
// every thread of the block.
__device__ void build_schedule_small(const int32_t* __restrict__ cu_g, int n, int H, int32_t* seq,
                                     int32_t* tiles, int32_t* nkv, int64_t* it_start, int32_t* tok0,
                                     int32_t* len, int32_t* cu) {
    // the offsets are staged in LDS once, so the O(n) rank loop below makes
    // no global loads
    for (int i = threadIdx.x; i <= n; i += blockDim.x) cu[i] = cu_g[i];
    __syncthreads();
    for (int s = threadIdx.x; s < n; s += blockDim.x) {
        const int Ls = cu[s + 1] - cu[s];
        const int cs = octave_class(Ls);
        int rank = 0;
        for (int i = 0; i < n; ++i) {
            const int ci = octave_class(cu[i + 1] - cu[i]);
            rank += (ci > cs) || (ci == cs && i < s);
        }
        seq[rank] = s;
        tiles[rank] = (Ls + kBM - 1) / kBM;
        nkv[rank] = (Ls + kBN - 1) / kBN;
        tok0[rank] = cu[s];
        len[rank] = Ls;
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

// Schedule of a pack of any size in O(n / 256 + 256) per thread: a stable
// counting sort on the octave class.  Thread t owns the contiguous index
// range [t*per, (t+1)*per); its per-class counts, prefix-summed over the
// threads, give every sequence its rank in (descending class, index) order.
constexpr int kSchedThreads = 256;
__global__ __launch_bounds__(kSchedThreads) void attn_schedule_kernel(const int32_t* __restrict__ cu, int n,
                                                                      int H, unsigned char* __restrict__ ws) {
    __shared__ int cnt[kSchedThreads][kOctaves];
    __shared__ int start[kOctaves];
    __shared__ int64_t part[kSchedThreads];
    int32_t* ints = reinterpret_cast<int32_t*>(ws + 8);
    int32_t* seq = ints + 1;
    int32_t* tiles = ints + 1 + n;
    int32_t* nkv = ints + 1 + 2 * n;
    int64_t* pre = reinterpret_cast<int64_t*>(ws + sched_prefix_off(n));
    const int tid = threadIdx.x;
    const int per = (n + kSchedThreads - 1) / kSchedThreads;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
#pragma unroll
    for (int c = 0; c < kOctaves; ++c) cnt[tid][c] = 0;
    for (int s = s0; s < s1; ++s) ++cnt[tid][octave_class(cu[s + 1] - cu[s])];
    __syncthreads();
    if (tid < kOctaves) {                 // exclusive prefix over the threads, per class
        int acc = 0;
        for (int t = 0; t < kSchedThreads; ++t) {
            const int v = cnt[t][tid];
            cnt[t][tid] = acc;
            acc += v;
        }
        start[tid] = acc;                 // class total for now
    }
    __syncthreads();
    if (tid == 0) {                       // class starts, highest class first
        int acc = 0;
        for (int c = kOctaves - 1; c >= 0; --c) {
            const int v = start[c];
            start[c] = acc;
            acc += v;
        }
    }
    __syncthreads();
    for (int s = s0; s < s1; ++s) {
        const int L = cu[s + 1] - cu[s];
        const int c = octave_class(L);
        const int r = start[c] + cnt[tid][c]++;
        seq[r] = s;
        tiles[r] = (L + kBM - 1) / kBM;
        nkv[r] = (L + kBN - 1) / kBN;
    }
    __threadfence_block();
    __syncthreads();
    // exclusive prefix of tiles*H*nkv over the ranks
    int64_t sum = 0;
    for (int r = s0; r < s1; ++r) sum += int64_t(tiles[r]) * H * nkv[r];
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int64_t acc = 0;
        for (int t = 0; t < kSchedThreads; ++t) {
            const int64_t v = part[t];
            part[t] = acc;
            acc += v;
        }
        pre[n] = acc;
        *reinterpret_cast<int64_t*>(ws) = acc;
        ints[0] = n;
    }
    __syncthreads();
    int64_t acc = part[tid];
    for (int r = s0; r < s1; ++r) {
        pre[r] = acc;
        acc += int64_t(tiles[r]) * H * nkv[r];
    }
}

// Schedule of this call: built in LDS for small packs, else the prologue's.
struct SchedLds {
    int32_t seq[kInlineSeqs], tiles[kInlineSeqs], nkv[kInlineSeqs], tok0[kInlineSeqs], len[kInlineSeqs];
    int32_t cu[kInlineSeqs + 1];
    int64_t it_start[kInlineSeqs + 1];
};

__device__ Sched get_schedule(const int32_t* cu, int n, int H, const unsigned char* ws, SchedLds& lds) {
    Sched s;
    s.n = n;
    if (n <= kInlineSeqs) {
        build_schedule_small(cu, n, H, lds.seq, lds.tiles, lds.nkv, lds.it_start, lds.tok0, lds.len, lds.cu);
        s.tok0 = lds.tok0;
        s.len = lds.len;
        s.seq = lds.seq;
        s.tiles = lds.tiles;
        s.nkv = lds.nkv;
        s.it_start = lds.it_start;
    } else {
        const int32_t* ints = reinterpret_cast<const int32_t*>(ws + 8);
        s.tok0 = nullptr;
        s.len = nullptr;
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

// LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)(p)));
}

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at LDS
// address lds + 16*i; offsets past the resource's range deposit zeros.
// Written in assembly so that the compiler does not treat it as an LDS write
// (it would then wait for all outstanding loads before every transposed LDS
// read); its completion is awaited explicitly with vmcnt.  lds and soff are
// wavefront-uniform.  The load gets the five wait states a VMEM read of an
// SGPR needs after a VALU (readfirstlane) wrote it, which the compiler cannot
// provide for an instruction inside assembly; they also cover the one a
// direct load needs after M0 is written.
__device__ __forceinline__ void dma16_asm(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16, lane layout as lds_read_tr16_b64)
// at LDS byte address a.
__device__ __forceinline__ s16x4_t lds_tr16_at(uint32_t a) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(uintptr_t(a)));
}

// vmcnt waits (expcnt and lgkmcnt unconstrained); vmcnt is 6 bits, split
// over bits [3:0] and [15:14] of the immediate.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

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
__global__ __launch_bounds__(Tile<D>::THREADS, 1) void attn_fwd_kernel(KParams p) {
    using TL = Tile<D>;
    constexpr int KK = TL::KK, EB = TL::EB, NI_W = TL::NI_W, NS = TL::NS, NP = TL::NP, NB = TL::NB;
    constexpr int kWaves = TL::WAVES, kRows = TL::ROWS_W;
    // Score tile of one 32-key step for the lane's query row: 16 keys per
    // lane, for each 32-row block of the wavefront.
    typedef f32x16_t Scores[NB];
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ SchedLds sched_lds;
    __shared__ int redo_flag[kWaves];

    const Sched sch = get_schedule(p.cu, p.n_seq, p.H, p.ws, sched_lds);
    const int g = logical_wg(blockIdx.x, p.G);
    const int64_t it_begin = range_begin(sch.W, g, p.G);
    const int64_t it_end = range_begin(sch.W, g + 1, p.G);
    unsigned char* const partials = p.ws + sched_bytes(p.n_seq);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int64_t ld = p.ld_qkv;
    const uint32_t row_bytes = uint32_t(ld) * 2u;
    const float c = p.scale_log2;

    // LDS: K stages 0 .. kKStages-1, then V stages 0 .. kVStages-1.
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    auto kstage = [&](int s) -> uint32_t { return uint32_t(s * TL::TILE_BYTES); };
    auto vstage = [&](int s) -> uint32_t { return uint32_t(s * TL::TILE_BYTES); };

    // ---- direct-load source offsets (same for every tile) ------------------
    // Instruction n of a tile fills LDS units [64n, 64n+64) of the stage;
    // lane i fills unit 64n+i = (row, stored unit) and so fetches the row's
    // unit (stored unit ^ swizzle).  Wavefront w issues instructions
    // w, w + kWaves, ...
    uint32_t k_voff[NI_W], v_voff[NI_W];
#pragma unroll
    for (int j = 0; j < NI_W; ++j) {
        const int u = 64 * (wave + kWaves * j) + lane;
        const int row = u / TL::U, su = u % TL::U;
        k_voff[j] = uint32_t(row) * row_bytes + 16u * uint32_t(su ^ swz_k<D>(row));
        v_voff[j] = uint32_t(row) * row_bytes + 16u * uint32_t(su ^ swz_v<D>(row));
    }
    // ---- LDS read offsets ----------------------------------------------------
    // K fragment kk (d-step kk): row l32, unit 2 kk + hlf, stored at
    // (2 kk + hlf) ^ swz(l32), i.e. at byte k_rd ^ 32 kk.
    const uint32_t k_rd = uint32_t(l32 * TL::ROW_BYTES + 16 * (hlf ^ swz_k<D>(l32)));
    // V^T fragment gi (16-key chunk gi / EB, output block m = gi % EB) via two
    // transposed reads: in each 16-lane group lane j addresses row
    // 16 cc + 4 hlf + j/4 (+8 for the second read) at dims
    // 32m + 16*(group&1) + 4*(j&3); lane i then receives dim 32m + (lane&31)
    // for 4 consecutive keys.  The swizzle of those rows depends only on j/4
    // and is a multiple of 4 units, so output block m is stored at
    // byte v_rd ^ 64 m.
    const uint32_t v_rd = [&] {
        const int vrow = 4 * hlf + ((lane & 15) >> 2);
        const int vu = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        return uint32_t(vrow * TL::ROW_BYTES + 16 * (vu ^ swz_v<D>(vrow)) + 8 * (lane & 1));
    }();
    // Per-lane LDS byte addresses of the fragments in stage 0 of each ring,
    // kept in registers (opaque to the compiler, which would otherwise
    // recompute them before every read): a stage and a key chunk then add
    // only an immediate offset (every such offset stays below 64 KB).
    uint32_t ka[KK], va[EB];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        ka[kk] = lds0 + (k_rd ^ uint32_t(32 * kk));
        asm volatile("" : "+v"(ka[kk]));
    }
#pragma unroll
    for (int m = 0; m < EB; ++m) {
        va[m] = lds0 + kKStages * TL::TILE_BYTES + (v_rd ^ uint32_t(64 * m));
        asm volatile("" : "+v"(va[m]));
    }
    typedef __attribute__((address_space(3))) const bf16x8_t* lds_b128_ptr;
    // kb, vb: byte offsets of a stage from the start of its ring
    auto kfrag = [&](uint32_t kb, int kk) -> bf16x8_t {
        return *reinterpret_cast<lds_b128_ptr>(uintptr_t(ka[kk] + kb));
    };
    auto vfrag = [&](uint32_t vb, int gi) -> bf16x8_t {
        const uint32_t a = va[gi % EB] + vb + (gi / EB) * 16 * TL::ROW_BYTES;
        const s16x4_t lo = lds_tr16_at(a);
        const s16x4_t hi = lds_tr16_at(a + 8 * TL::ROW_BYTES);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    bool first_segment = true;
    for (int64_t it = it_begin; it < it_end;) {
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
        const bool first_piece = it == it_begin;
        const int head = tile / nt;
        const int qtile = tile - head * nt;
        // the sequence's first token and length (from the LDS schedule when
        // there is one: no global load on the segment's critical path)
        const int64_t tok0 = __builtin_amdgcn_readfirstlane(sch.tok0 ? sch.tok0[rank] : p.cu[seq]);
        const int L = sch.len ? __builtin_amdgcn_readfirstlane(sch.len[rank])
                              : __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);
        // Key step j of a tile processes key tile (j + nkv - 1) % nkv: the
        // sequence's last key tile, the only one with keys past the end
        // (masked when L is not a multiple of kBN), comes first, so only the
        // first step of a tile's first segment ever masks and the step loop
        // has no mask branch (the softmax does not depend on key order).
        const bool mask_first = kv0 == 0 && (L % kBN) != 0;
        it += kv1 - kv0;
        const int n = kv1 - kv0;

        // Buffer resources over this sequence's rows of the head: loads of
        // rows at or past L return zeros (ragged q-tile and last key tile).
        const uint64_t seq_bytes = uint64_t(L) * uint64_t(ld) * 2u;
        const int64_t head_off = tok0 * ld + int64_t(head) * D;
        const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + head_off, seq_bytes);
        const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + head_off, seq_bytes);
        const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + head_off, seq_bytes);
        // Scalar offset of key step j's tile, or an out-of-range offset for a
        // step this segment does not take (the load then deposits zeros
        // without touching memory; an offset that still lands inside a
        // sequence of more than 2 GiB reads valid rows into a stage nobody
        // reads).
        auto tile_soff = [&](int j) -> uint32_t {
            const int kt = j == 0 ? nkv - 1 : j - 1;
            return j < kv1 ? uint32_t(kt) * uint32_t(kBN) * row_bytes : kOutOfRange;
        };
        // ... for a key step j >= 1 (all steps the step loop loads)
        auto tile_soff_pos = [&](int j) -> uint32_t {
            return j < kv1 ? uint32_t(j - 1) * uint32_t(kBN) * row_bytes : kOutOfRange;
        };
        // The step loop runs its steps in groups of kRing with every ring
        // position a compile-time constant (so LDS stage addresses are
        // immediates); the m % kRing steps that do not fill a group run first,
        // with run-time ring positions.  Tile kv0 is placed at ring position
        // ph0 so that the groups start at position 0 and the last step of
        // the segment (tile kv1 - 1) sits at position 0.
        const int m_steps = n - 1;     // steps followed by another step
        const int r_steps = m_steps & (kRing - 1);
        const int ph0 = (kRing - r_steps) & (kRing - 1);
        auto dma_k = [&](int stage, uint32_t so, int j) {
            dma16_asm(k_rs, lds0 + stage * TL::TILE_BYTES + 1024 * (wave + kWaves * j), k_voff[j], so);
        };
        auto dma_v = [&](int stage, uint32_t so, int j) {
            dma16_asm(v_rs, lds0 + (kKStages + stage) * TL::TILE_BYTES + 1024 * (wave + kWaves * j),
                      v_voff[j], so);
        };

        // The previous segment's LDS reads are done before any of its stages
        // is refilled.  (Its last direct loads need no wait: a wavefront's
        // loads land in issue order, so they land before this segment's.)
        if (!first_segment) __syncthreads();
        first_segment = false;

        // Q^T fragments (B operand) of the row blocks, kept in registers.
        bf16x8_t qf[NB][KK];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int qrow = qtile * kBM + wave * kRows + 32 * b + l32;
            const uint32_t qoff = uint32_t(qrow) * row_bytes + 16u * hlf;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                qf[b][kk] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, qoff, 32u * kk));
        }

        // Keys at or past L of the score tile s of the sequence's last key
        // tile: -inf.
        auto mask_scores = [&](Scores& s) {
            const int lim = L - (nkv - 1) * kBN - 4 * hlf;   // key offsets >= lim are past the end
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + (r & 3) >= lim) s[b][r] = -INFINITY;
        };
        // S = K Q^T of the K tile in LDS at kb (no overlapped work).
        auto scores = [&](Scores& s, uint32_t kb) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t f = kfrag(kb, kk);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[b][kk], kk == 0 ? f32x16_t{} : s[b], 0, 0, 0);
            }
        };

        // The reference max m of each row (log2 units) is fixed by the first
        // key step of the segment, so p = 2^(x - m) may exceed 1 on later
        // steps; numerator and denominator share m, so the result is the same
        // softmax.  No step checks anything: at the end, a row sum above
        // 2^64 (or not finite) means that some p may have overflowed, and the
        // whole workgroup then redoes the segment once with every reference
        // max preset to the row's exact maximum over the segment's keys
        // (found by a scores-only pass), after which every p <= 1.  So the
        // output accumulators are only ever written by MFMAs, and the step
        // loop carries no max or rescale work.
        bool preset = false;
        float m_pre[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) m_pre[b] = -INFINITY;
        for (;;) {
            if (preset) {
                // the failed attempt's loads have landed and its LDS reads
                // are done before the scores-only pass refills K stage 0
                wait_vm<0>();
                __syncthreads();
                // exact row maxima over key steps kv0 .. kv1-1, one tile at a
                // time through K stage 0
                Scores sp;
                for (int j = kv0; j < kv1; ++j) {
#pragma unroll
                    for (int jj = 0; jj < NI_W; ++jj) dma_k(0, tile_soff(j), jj);
                    wait_vm<0>();
                    __syncthreads();
                    scores(sp, kstage(0));
                    if (j == 0 && mask_first) mask_scores(sp);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        float mxb = sp[b][0];
#pragma unroll
                        for (int r = 1; r < 16; ++r) mxb = fmaxf(mxb, sp[b][r]);
                        m_pre[b] = fmaxf(m_pre[b], half_max(mxb) * c);
                    }
                    __syncthreads();
                }
            }
            // Tile kv0+i lives in stage (ph0 + i) mod kRing of each ring.  The
            // prologue loads K of tiles kv0 .. kv0+7 and V of tiles kv0 ..
            // kv0+6 in the order they are first read: K0 K1 K2 V0 (before step
            // 0), then K(i+2) and V(i) for step i = 1 .. 5, then V6, so that
            // the constant vmcnt wait at the end of each step also covers them.
            {
                auto pk = [&](int i) {
#pragma unroll
                    for (int j = 0; j < NI_W; ++j) dma_k((ph0 + i) & (kRing - 1), tile_soff(kv0 + i), j);
                };
                auto pv = [&](int i) {
#pragma unroll
                    for (int j = 0; j < NI_W; ++j) dma_v((ph0 + i) & (kRing - 1), tile_soff(kv0 + i), j);
                };
                pk(0); pk(1); pk(2); pv(0);
#pragma unroll
                for (int i = 1; i <= 5; ++i) { pk(i + 2); pv(i); }
                pv(6);
            }

            f32x16_t o[NB][EB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int m = 0; m < EB; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][m][r] = 0.f;
            float m_run[NB], negm[NB], lsum[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) lsum[b] = 0.f;

            bf16x8_t kf[kPfK], vf[kPfV];
            bf16x8_t pf[NB][2];
            Scores h0, h1;

            // K0 K1 K2 V0 have landed (11 later prologue tiles may be in flight)
            wait_vm<11 * NI_W>();
            __syncthreads();

            // ---- phase 1: S(t+1) = K(t+1) Q^T || p = exp2(x(t)) (kExp) ------
            // Slot i issues S MFMA i (d-step i / NB, row block i % NB: each K
            // fragment feeds the NB row blocks) and the exponentials of x
            // elements [E i, E i + E) (element e: row block e/16, register
            // e%16); the bf16 rounding and row sums of slot i's pairs run in
            // slot i+1.  The first V fragments of phase 2 are read in the last
            // slots.
            auto phase1 = [&]<bool kS>(Scores& x, Scores& s, uint32_t kb, uint32_t vb) {
                constexpr int E = 16 * NB / NS;
                static_for<NS + 1>([&](auto SI) {
                    constexpr int sl = SI;
                    if constexpr (kS && sl < NS) {
                        constexpr int kk = sl / NB, b = sl % NB;
                        if constexpr (kk == 0)
                            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % kPfK], qf[b][kk], f32x16_t{}, 0, 0, 0);
                        else
                            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % kPfK], qf[b][kk], s[b], 0, 0, 0);
                        if constexpr (b == NB - 1 && kk + kPfK < KK) kf[kk % kPfK] = kfrag(kb, kk + kPfK);
                    }
                    if constexpr (sl > 0) {
                        // bf16 rounding of the previous slot's pairs
#pragma unroll
                        for (int i = 0; i < E; i += 2) {
                            const int e = E * (sl - 1) + i;
                            const int b = e / 16, r = e % 16;
                            const uint32_t w = pack_bf16x2(x[b][r], x[b][r + 1]);
                            const int cc = r / 8, dw = (r % 8) / 2;
                            u32x4_t u = __builtin_bit_cast(u32x4_t, pf[b][cc]);
                            u[dw] = w;
                            pf[b][cc] = __builtin_bit_cast(bf16x8_t, u);
                        }
                    }
                    if constexpr (sl < NS) {
#pragma unroll
                        for (int i = 0; i < E; ++i) {
                            const int e = E * sl + i;
                            x[e / 16][e % 16] = __builtin_amdgcn_exp2f(x[e / 16][e % 16]);
                        }
                    }
                    if constexpr (sl >= NS + 1 - kPfV) vf[sl - (NS + 1 - kPfV)] = vfrag(vb, sl - (NS + 1 - kPfV));
                    __builtin_amdgcn_sched_barrier(0);
                });
            };

            // ---- phase 2: O += V(t)^T P(t)^T || front half of softmax(t+1) --
            // Slot i issues PV MFMA i (chunk i / (NB EB), output block
            // (i / NB) % EB, row block i % NB: each V fragment feeds the NB
            // row blocks).  With
            // kNext the slots also carry the front half of the next tile's
            // softmax: the row maxima of S(t+1), the raise check and
            // x(t+1) = S(t+1) c - m, in place; they issue the step's direct
            // loads (K of tile t+kKStages, V of tile t+kVStages-1) in slots
            // 1 .. 2 NI_W and read the first K fragments of the next phase 1
            // in the last slots.
            auto phase2 = [&]<bool kNext>(Scores& s, Scores& pr, uint32_t vb, uint32_t kb_next, int t,
                                          int kdst, int vdst) {
                constexpr int NITEMS = kNext ? 16 * NB : 0;   // x = S c - m, in place
                constexpr int NSUMS = 8 * NB;                  // pairs of p(t) added to the row sums
                const uint32_t so_k = tile_soff_pos(t + kKStages), so_v = tile_soff_pos(t + kVStages - 1);
                auto item = [&](auto II) {
                    constexpr int e = II;
                    constexpr int b = e / 16, r = e % 16;
                    s[b][r] = __builtin_fmaf(s[b][r], c, negm[b]);
                };
                static_for<NP>([&](auto SI) {
                    constexpr int sl = SI;
                    constexpr int gi = sl / NB, b = sl % NB, cc = gi / EB, m = gi % EB;
                    o[b][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[gi % kPfV], pf[b][cc], o[b][m], 0, 0, 0);
                    if constexpr (b == NB - 1 && gi + kPfV < TL::NV_FR) vf[gi % kPfV] = vfrag(vb, gi + kPfV);
                    if constexpr (kNext && sl >= 1 && sl <= NI_W) dma_k(kdst, so_k, sl - 1);
                    if constexpr (kNext && sl > NI_W && sl <= 2 * NI_W) dma_v(vdst, so_v, sl - NI_W - 1);
                    constexpr int lo = NITEMS * sl / NP, hi = NITEMS * (sl + 1) / NP;
                    static_for<hi - lo>([&](auto JI) { item(std::integral_constant<int, lo + int(JI)>{}); });
                    constexpr int slo = NSUMS * sl / NP, shi = NSUMS * (sl + 1) / NP;
                    static_for<shi - slo>([&](auto JI) {
                        constexpr int e = 2 * (slo + int(JI)), b = e / 16, r = e % 16;
                        lsum[b] += pr[b][r] + pr[b][r + 1];
                    });
                    if constexpr (kNext && sl >= NP - kPfK) kf[sl - (NP - kPfK)] = kfrag(kb_next, sl - (NP - kPfK));
                    __builtin_amdgcn_sched_barrier(0);
                });
            };

            // ---- first tile: S(kv0), its row maxima and x(kv0) -------------
            scores(h0, kstage(ph0));
            if (mask_first) mask_scores(h0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float mxb = fmaxf(h0[b][0], h0[b][1]);
#pragma unroll
                for (int r = 2; r < 16; r += 2) mxb = fmaxf(mxb, fmaxf(h0[b][r], h0[b][r + 1]));
                m_run[b] = fmaxf(half_max(mxb) * c, m_pre[b]);
                negm[b] = -m_run[b];
#pragma unroll
                for (int r = 0; r < 16; ++r) h0[b][r] = __builtin_fmaf(h0[b][r], c, negm[b]);
            }
#pragma unroll
            for (int i = 0; i < kPfK; ++i) kf[i] = kfrag(kstage((ph0 + 1) & (kRing - 1)), i);
            // every wavefront is done with K of tile kv0 before step 0 refills it
            __syncthreads();

            // ---- key steps ---------------------------------------------------
            // Step t (tile t at ring position ph) reads K(t+1) and V(t),
            // refills the K stage of tile t with tile t+8 and the V stage of
            // tile t-1 with tile t+7, waits until the loads it and the other
            // steps issued kSlack steps before or earlier have landed, and
            // passes the step barrier.  A tile is read no earlier than the step
            // after the barrier that published it, and a stage is refilled only
            // after the barrier that ended its last reads.  x(t) and S(t+1)
            // alternate between h0 and h1 (even ring positions read x from h0).
            auto step = [&](Scores& x, Scores& s, int t, int ph) {
                const int ks = (ph + 1) & (kRing - 1);       // K stage of tile t+1
                const int ks2 = (ph + 2) & (kRing - 1);      // K stage of tile t+2
                const int vd = (ph + kRing - 1) & (kRing - 1);  // V stage of tile t-1
                phase1.template operator()<true>(x, s, kstage(ks), vstage(ph));
                phase2.template operator()<true>(s, x, vstage(ph), kstage(ks2), t, ph, vd);
                wait_vm<2 * NI_W * kSlack>();
                __syncthreads();
            };
            int i = 0;
            for (; i < r_steps; ++i) {
                step(h0, h1, kv0 + i, (ph0 + i) & (kRing - 1));
#pragma unroll
                for (int b = 0; b < NB; ++b) h0[b] = h1[b];
            }
            for (; i < m_steps; i += kRing) {
                static_for<kRing>([&](auto P) {
                    constexpr int ph = P;
                    if constexpr (ph % 2 == 0) step(h0, h1, kv0 + i + ph, ph);
                    else step(h1, h0, kv0 + i + ph, ph);
                });
            }
            // the segment's last tile, at ring position 0
            phase1.template operator()<false>(h0, h0, kstage(1), vstage(0));
            phase2.template operator()<false>(h0, h0, vstage(0), kstage(2), kv1, 0, 0);

            // ---- redo decision (workgroup-wide) --------------------------------
            // A row sum is at least every one of its terms, so a sum within
            // the limit (and finite) shows that no probability overflowed.
            if (!preset) {
                bool big = false;
#pragma unroll
                for (int b = 0; b < NB; ++b) big |= !(lsum[b] <= kSumLimit);
                const bool raised = __builtin_amdgcn_ballot_w64(big) != 0;
                if (lane == 0) redo_flag[wave] = raised;
                __syncthreads();
                bool any = false;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) any |= redo_flag[w] != 0;
                if (__builtin_amdgcn_readfirstlane(any)) {
                    preset = true;
                    continue;
                }
            }

            // ---- epilogue --------------------------------------------------
            float l_tot[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) l_tot[b] = half_sum(lsum[b]);
            if (kv0 == 0 && kv1 == nkv) {
                // whole tile: normalise and store O (bf16) and the LSE
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int qrow = qtile * kBM + wave * kRows + 32 * b + l32;
                    if (qrow < L) {
                        const float inv = 1.0f / l_tot[b];
                        uint16_t* op = p.o + (tok0 + qrow) * p.ld_o + int64_t(head) * D + 4 * hlf;
#pragma unroll
                        for (int m = 0; m < EB; ++m)
#pragma unroll
                            for (int gq = 0; gq < 4; ++gq) {
                                u32x2_t val;
                                val[0] = pack_bf16x2(o[b][m][4 * gq] * inv, o[b][m][4 * gq + 1] * inv);
                                val[1] = pack_bf16x2(o[b][m][4 * gq + 2] * inv, o[b][m][4 * gq + 3] * inv);
                                *reinterpret_cast<u32x2_t*>(op + 32 * m + 8 * gq) = val;
                            }
                        if (p.lse != nullptr && hlf == 0)
                            p.lse[int64_t(head) * p.T + tok0 + qrow] =
                                m_run[b] * 0.69314718055994531f + logf(l_tot[b]);
                    }
                }
            } else {
                // piece of a tile shared with other workgroups: partial in slot
                // 2g (this workgroup's first segment) or 2g+1 (its last)
                unsigned char* slot = partials + size_t(2 * g + (first_piece ? 0 : 1)) * TL::SLOT_BYTES;
                float* acc = reinterpret_cast<float*>(slot);
                float* ml = reinterpret_cast<float*>(slot + size_t(kBM) * D * 4);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int row = wave * kRows + 32 * b + l32;
#pragma unroll
                    for (int m = 0; m < EB; ++m)
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const f32x4_t val = {o[b][m][4 * gq], o[b][m][4 * gq + 1], o[b][m][4 * gq + 2],
                                                 o[b][m][4 * gq + 3]};
                            *reinterpret_cast<f32x4_t*>(acc + row * D + 32 * m + 8 * gq + 4 * hlf) = val;
                        }
                    if (hlf == 0) {
                        ml[row] = m_run[b];
                        ml[kBM + row] = l_tot[b];
                    }
                }
            }
            break;
        }
    }
    // no direct load may still be in flight when the wavefront ends
    wait_vm<0>();
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
    auto ml_at = [&](int i) { return reinterpret_cast<const float*>(slot_at(i) + size_t(kBM) * D * 4); };

    // per row: the reference max M over the pieces and 1 / total weight.
    // Pieces are read two at a time with all their loads issued together
    // (one memory round trip per pair instead of one per load); the sums
    // keep the order of a piece-by-piece pass.
    __shared__ float row_m[kBM], row_inv[kBM];
    const int tid = threadIdx.x;
    if (tid < kBM) {
        float M = -INFINITY, lt = 0.f;
        for (int i = 0; i < ns; i += 2) {
            const bool has1 = i + 1 < ns;
            const float m0 = ml_at(i)[tid], l0 = ml_at(i)[kBM + tid];
            const float m1 = has1 ? ml_at(i + 1)[tid] : -INFINITY;
            const float l1 = has1 ? ml_at(i + 1)[kBM + tid] : 0.f;
            const float Mn = fmaxf(M, fmaxf(m0, m1));
            lt = lt * exp2f(M - Mn) + exp2f(m0 - Mn) * l0;
            if (has1) lt += exp2f(m1 - Mn) * l1;
            M = Mn;
        }
        row_m[tid] = M;
        row_inv[tid] = 1.0f / lt;
        const int qrow = qtile * kBM + tid;
        if (p.lse != nullptr && qrow < L) p.lse[int64_t(head) * p.T + tok0 + qrow] = M * 0.69314718055994531f + logf(lt);
    }
    __syncthreads();

    // weighted sum of the pieces over the tile's 16-byte chunks (4 fp32) in
    // memory order (consecutive lanes read consecutive chunks), the chunks
    // of a pair of pieces loaded together
    constexpr int kRowChunks = D / 4;
    constexpr int kChunks = kBM * kRowChunks;
    constexpr int kPer = kChunks / kFixThreads;
    static_assert(kChunks % kFixThreads == 0, "whole chunks per thread");
    float acc[kPer][4];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
    // a thread's chunks in rounds of kRound, so that a pair's loads (2 x
    // kRound x 16 bytes) stay within the 128 registers of 1024 threads
    constexpr int kRound = kPer > 4 ? 4 : kPer;
    static_assert(kPer % kRound == 0, "whole rounds of chunks");
#pragma unroll
    for (int j0 = 0; j0 < kPer; j0 += kRound) {
        for (int i = 0; i < ns; i += 2) {
            f32x4_t raw[2][kRound];
            float w[2][kRound];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const bool has = i + k < ns;
                const unsigned char* sl = slot_at(has ? i + k : i);
                const float* ml = ml_at(has ? i + k : i);
#pragma unroll
                for (int j = 0; j < kRound; ++j) {
                    const int cidx = tid + kFixThreads * (j0 + j);
                    const int row = cidx / kRowChunks;
                    raw[k][j] = reinterpret_cast<const f32x4_t*>(sl)[cidx];
                    w[k][j] = has ? exp2f(ml[row] - row_m[row]) : 0.f;
                }
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (i + k >= ns) break;
#pragma unroll
                for (int j = 0; j < kRound; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[j0 + j][e] += w[k][j] * raw[k][j][e];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int cidx = tid + kFixThreads * j;
        const int row = cidx / kRowChunks;
        const int qrow = qtile * kBM + row;
        if (qrow >= L) continue;
        const float inv = row_inv[row];
        u32x2_t val;
        val[0] = pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv);
        val[1] = pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv);
        *reinterpret_cast<u32x2_t*>(p.o + (tok0 + qrow) * p.ld_o + int64_t(head) * D + 4 * (cidx % kRowChunks)) = val;
    }
}

std::atomic<int> g_grid_override{0};

// Persistent workgroups of a call: one per CU unless a test overrides it.
int attn_grid() {
    const int o = g_grid_override.load(std::memory_order_relaxed);
    return o > 0 ? o : device_cu_count();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
    const int G = attn_grid();
    if (G <= 0) return hipErrorInvalidDevice;
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    if (a.n_seq > kInlineSeqs) {
        hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a.cu_seqlens,
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
    hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(G), dim3(Tile<D>::THREADS), smem, stream, p);
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
    int G = attn_grid();
    if (G <= 0) G = 256;   // no device visible: size for an MI355X
    const size_t slot = D == 64 ? Tile<64>::SLOT_BYTES : Tile<128>::SLOT_BYTES;
    return sched_bytes(n) + size_t(2) * G * slot;
}

void set_attn_fwd_grid(int g) { g_grid_override.store(g, std::memory_order_relaxed); }

// ---------------------------------------------------------------------------
// Allocation-free forward.  Its workspace (schedule and partial slots, none
// of which needs to start zeroed) is this file-scope array: one copy per GPU,
// allocated with the code object and held until the process ends.  Host code
// never passes the array's name to a kernel (that is a host-side stand-in);
// it looks up the device address once per device and passes that.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kAttnNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;

// Device address of the current device's scratch array.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_varlen_attn_fwd_noalloc(const AttnArgs& args, hipStream_t stream) {
    void* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return e;
    AttnArgs a = args;
    a.workspace = p;
    a.workspace_bytes = kAttnNoAllocScratchBytes;
    return launch_varlen_attn_fwd(a, stream);
}

hipError_t launch_varlen_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_d<128>(a, stream);
    return launch_d<64>(a, stream);
}

}  // namespace mf
