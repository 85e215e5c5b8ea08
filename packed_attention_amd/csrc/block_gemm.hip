// Block projections around the attention (gfx950): the QKV projection of the
// adaLN-modulated residual stream with the rotary embedding of q and k as its
// epilogue, and the out projection with the gated residual as its epilogue.
//
// The pages fuse the adaptive normalisation, rotary embedding and gating /
// residual chains with the operators around them (picx.dev summary of
// Mage-Flow, Methodology > Training Infrastructure; gist.science "Resumo
// Tecnico: Mage-Flow", Metodologia > 3. Otimizacao de Nivel de Sistema >
// Kernels Fundidos); in an NR-MMDiT block (picx.dev, Methodology >
// Native-Resolution MMDiT) those operators are these two projections.
//
//   u   = LN(x) * (1 + scale[m(t)]) + shift[m(t)]        (x: [T][C])
//   qkv = u W_qkv^T,  q' = RoPE(q), k' = RoPE(k), v       (W_qkv: [3C][C])
//   y   = x + gate[m(t)] * (o W_o^T)                      (W_o: [C][C])
//
// Design (MI355X, CDNA4):
//  * adaln_kernel: one wavefront per token row, LayerNorm statistics in fp32
//    (two passes over registers), the modulated row rounded to bf16 into the
//    caller's workspace.  The modulation is not recomputed inside the GEMM:
//    each activation element meets every 256-feature tile of the weight
//    (36 of them for the QKV projection at C = 3072), so a K-loop prologue
//    would cost ~4.5 VALU instructions per element per tile, about half of
//    the MFMA time, against 2*T*C*2 bytes of HBM traffic for writing the
//    modulated rows once and reading them back.
//  * gemm_kernel<MODE>: out^T = W act^T with v_mfma_f32_32x32x16_bf16, both
//    operands K-contiguous (weights [N][K] as stored, activations [T][K]), so
//    every MFMA fragment is one 16-byte LDS read.  A workgroup computes 256
//    features x 256 tokens with 8 wavefronts (2 per SIMD, 64 features x 128
//    tokens each, 128 accumulator registers).  K advances in steps of 64
//    through two LDS stages filled by direct global->LDS loads (no staging
//    registers); LDS rows are 128 bytes with their 16-byte chunks swizzled,
//    so the fragment reads are conflict-free without padding.  Each step's
//    one barrier sits before the MFMAs of its last K sub-step, so the next
//    step's first fragments and the loads two steps ahead are issued while
//    those MFMAs run, and scheduling groups keep every sub-step's fragment
//    reads one sub-step ahead of their MFMAs (two fragment sets).  Measured
//    on MI355X (the sustained rates of the same loop without global loads
//    and with them from L2 are within 2% of each other, and the barrier
//    alone costs nothing there), the step takes ~2450 cycles against 2048 of
//    MFMA issue; the rest comes with the loads from the memory system.
//    A four-wavefront layout (128 x 128 per wavefront, 256 accumulators in
//    AGPRs, one wavefront per SIMD) reads a third less LDS but measured 25%
//    slower: one wavefront per SIMD leaves no second wavefront to issue
//    MFMAs while the other waits.
//    Transposed output: each lane holds one token and 16 features, so the
//    RoPE pairs (adjacent features) sit in one lane.
//  * Rotation table: the modulation pass (or, without modulation, a small
//    kernel) writes (cos, sin) of every head pair of every token once, T*D/2
//    fp32 pairs in the workspace.  The epilogue then turns a pair with one
//    load per two pairs and four multiply-adds, instead of forming the fp64
//    angle and the sine and cosine for each of the 3C/2 x T pairs again in
//    each of the 2C/256 q and k feature tiles (the per-pair angle work was
//    most of the epilogue's instructions).
//  * Out projection epilogue: the gated residual needs x and gate along the
//    features, while a lane holds one token, so the fp32 tile goes through
//    LDS in two halves and every global access is a 512-byte row segment;
//    the residual and gate rows are loaded before the staging.
//  * Tiles are numbered so that the tiles one XCD runs are consecutive and
//    share their weight tile (its L2 serves the re-reads).
//  * Sliced tail (QKV projection): one workgroup per CU, so the tiles run in
//    rounds of #CUs; when the last round is at most half full, each of its
//    tiles is cut into two (or four) token slices of 128 (64) tokens that
//    run side by side in the same launch (workgroups after the whole tiles'),
//    each with the whole K and its own epilogue: the round takes about half
//    (a quarter) of a tile's time and nothing is added afterwards.  (Run as
//    a second launch, the slices measured slower: 241 -> 256 us at the
//    1024^2 pack, the launch gap and the lost overlap with the last whole
//    tiles.)
//  * Ragged edges: buffer resources end at the last token / feature, so rows
//    past them read as zeros; the epilogue stores only rows inside.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kGW = 8;                     // wavefronts per workgroup
constexpr int kGT = 64 * kGW;
constexpr int kBF = 256;                   // features per tile
constexpr int kBT = 256;                   // tokens per tile
constexpr int kBK = 64;                    // K per step
constexpr int kChunks = kBK / 8;           // 16-byte chunks per LDS row (128 bytes, no padding)
constexpr int kRowB = 16 * kChunks;
constexpr int kStages = 2;
constexpr int kLdsB = kStages * (kBF + kBT) * kRowB;   // 128 KiB: two stages of a whole tile
constexpr int kRowsPerDma = 64 / kChunks;  // LDS rows one direct-load instruction fills
constexpr int kDmaW = kBF / kRowsPerDma;   // direct-load instructions of a stage that fill the weight rows
constexpr int kXcds = 8;
constexpr int kGroupF = 4;                 // feature tiles per group of the tile order
// The epilogue stages the bf16 output tile [tokens][kBF features] through the
// (then free) LDS stages.

// LDS rows are stored swizzled: chunk c of row r sits in slot c ^ sw(r),
// sw(r) = (r / 2) % 8.  The 16 lanes one LDS cycle serves read 16-byte
// chunks of 16 consecutive rows (two per 256-byte bank line), and the swizzle
// gives each of them its own 4 banks without padding.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

enum { kModeQkv = 0, kModeOut = 1 };

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it (a full __syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct GemmParams {
    const uint16_t* w;       // [N][K]
    const uint16_t* act;     // [T][K], token stride ld_act
    int64_t ld_act;
    int64_t T;
    int N, K;
    uint16_t* out;           // [T][N], token stride ld_out
    int64_t ld_out;
    // QKV: RoPE on the features below rope_limit (q and k), from the
    // rotation table: (cos, sin) of pair i of a head at token t in
    // rope_cs[t * D/2 + i]
    int rope_limit, D;
    const f32x2_t* rope_cs;
    // out projection: y = resid + gate[m] * acc
    const uint16_t* resid;
    const uint16_t* gate;
    const int32_t* mod_row;
    int n_rows;              // a row outside [0, n_rows) gates with zeros
    int tiles_t, tiles_f;
    // tail: tiles [n_full, tiles) run as `slices` token slices each
    int n_full, slices;
};

// The rotation table: for token t and pair i of a head (dims 2i, 2i+1 on
// the axis their block belongs to), cs[t * D/2 + i] = (cos, sin) of
// pos_axis(t) * theta_i.  The angle is formed in fp64 in turns and reduced to
// [-1/2, 1/2] before the hardware sine and cosine.
struct RopeTableParams {
    f32x2_t* cs;
    const int32_t* pos;
    int D, rope_f, rope_r;
    double theta_turns[64];
};

__device__ __forceinline__ void rope_table_row(const RopeTableParams& rp, int64_t t, int lane) {
    const int half = rp.D >> 1;
    for (int i = lane; i < half; i += kWave) {
        const int e = 2 * i;
        const int axis = e < rp.rope_f ? 0 : (e < rp.rope_f + rp.rope_r ? 1 : 2);
        const double turns = double(rp.pos[3 * t + axis]) * rp.theta_turns[i];
        const float f = float(turns - rint(turns));
        rp.cs[t * half + i] = f32x2_t{__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f)};
    }
}

// Shape of a tile of BT tokens (256: the whole tiles; 128 and 64: slices of
// the last round's tiles).  Wavefront (wf, wt) computes features
// 64 wf .. 64 wf + 63 and tokens kWT wt .. kWT wt + kWT - 1.
template <int BT>
struct Tile {
    static_assert(BT == 256 || BT == 128 || BT == 64, "tile tokens");
    static constexpr int kTB = BT / 64;                     // 32-token blocks per wavefront
    static constexpr int kWT = BT / 2;                      // tokens per wavefront
    static constexpr int kStageRows = kBF + BT;
    static constexpr int kStageB = kStageRows * kRowB;
    static constexpr int kDmaPerWave = kStageRows / kRowsPerDma / kGW;
    static_assert(kStageRows / kRowsPerDma % kGW == 0, "whole direct-load instructions");
    static_assert(2 * kStageB <= kLdsB && BT * kBF * 2 <= 2 * kStageB, "stages and output image fit");
};

// Logical tile -> (feature tile, token tile): groups of kGroupF feature
// tiles; consecutive tiles walk the group's feature tiles for one token tile,
// then the next token tile, so the tiles running together on an XCD share
// both operands' K slabs.
__device__ __forceinline__ void tile_of(const GemmParams& p, int lt, int& ft, int& tt) {
    const int gsz = kGroupF * p.tiles_t;
    const int grp = lt / gsz, rem = lt - grp * gsz;
    const int gf = min(kGroupF, p.tiles_f - grp * kGroupF);
    ft = grp * kGroupF + rem % gf;
    tt = rem / gf;
}

// Item b of n in an order where the items one XCD runs are consecutive
// (blockIdx round-robins over the XCDs).
__device__ __forceinline__ int xcd_order(int b, int n) {
    return n % kXcds == 0 ? (b % kXcds) * (n / kXcds) + b / kXcds : b;
}

// Wait until at most N of this wavefront's direct global->LDS loads are in
// flight (they complete in order); expcnt and lgkmcnt unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Epilogue of one tile from its fp32 accumulators (lane = token, register r
// of block fb = feature 8(r/4) + 4h + r%4 of the block).
//
// QKV projection: q and k pairs are turned by the table's rotation (register
// pair (4j + 2c, 4j + 2c + 1) is head pair hp + 4j + c, hp = (nblk mod D)/2
// + 2h, so one 16-byte table load serves two pairs), the values rounded to
// bf16 go to an LDS image of the output tile (rows = tokens, 512 bytes;
// 16-byte chunk c of row t in slot c ^ (t % 32), so the 8-byte writes of 32
// consecutive rows and the 16-byte reads along a row are both conflict-free)
// and out one 512-byte row segment per 32 lanes.
//
// Out projection: y = x + gate * acc needs x and gate along the features, so
// the fp32 tile goes through LDS in two halves of 128 tokens (rows of 1 KiB,
// 16-byte chunk c of row t in slot c ^ (t % 16)); each wavefront then takes
// whole rows, lane = 4 consecutive features, and every global load and store
// is a 512-byte row segment.
template <int MODE, int BT>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, f32x16_t (&acc)[2][Tile<BT>::kTB],
                                              const int f0, const int64_t t0, unsigned char* smem) {
    constexpr int kTB = Tile<BT>::kTB;
    constexpr int kWT = Tile<BT>::kWT;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int wf = wave & 3;
    const int wt = wave >> 2;
    if constexpr (MODE == kModeQkv) {
        // Table entries of the lane's token in each token block, one 16-byte
        // load per two pairs, double-buffered over the token blocks (rows
        // past T load row T - 1 and go unused); the first block's loads are
        // in flight across the barrier.
        f32x4_t cbuf[2][2][4];
        auto load_cs = [&](int buf, int tb) {
            const int64_t t = t0 + kWT * wt + 32 * tb + l32;
            const int64_t tc = t < p.T ? t : p.T - 1;
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                const int nblk = f0 + 64 * wf + 32 * fb;
                if (nblk < p.rope_limit) {
                    const int hp = ((nblk % p.D) >> 1) + 2 * hlf;
                    const f32x4_t* cs = reinterpret_cast<const f32x4_t*>(p.rope_cs + tc * (p.D >> 1) + hp);
#pragma unroll
                    for (int j = 0; j < 4; ++j) cbuf[buf][fb][j] = cs[2 * j];
                }
            }
        };
        load_cs(0, 0);
        lds_barrier();                     // every wavefront is done with the stages
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) {
            if (tb + 1 < kTB) load_cs((tb + 1) & 1, tb + 1);
            const int tl = kWT * wt + 32 * tb + l32;   // token row inside the tile
            const int64_t t = t0 + tl;
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                const int fl = 64 * wf + 32 * fb;      // first feature of the block inside the tile
                const int nblk = f0 + fl;
                f32x16_t& a = acc[fb][tb];
                if (nblk < p.rope_limit && t < p.T) {
                    const f32x4_t* c = cbuf[tb & 1][fb];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int r = 4 * j + 2 * h;
                            const float co = c[j][2 * h], sn = c[j][2 * h + 1];
                            const float x0 = a[r], x1 = a[r + 1];
                            a[r] = x0 * co - x1 * sn;
                            a[r + 1] = x0 * sn + x1 * co;
                        }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int f = fl + 8 * g + 4 * hlf;        // feature inside the tile
                    u32x2_t val;
                    val[0] = pack_bf16x2(a[4 * g], a[4 * g + 1]);
                    val[1] = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
                    const int slot = (f >> 3) ^ (tl & 31);
                    *reinterpret_cast<u32x2_t*>(smem + tl * 512 + 16 * slot + 8 * ((f >> 2) & 1)) = val;
                }
            }
        }
        lds_barrier();
        // rows 2 (i kGW + wave) + h, chunk l32: 32 lanes per 512-byte row segment
#pragma unroll 4
        for (int i = 0; i < BT / (2 * kGW); ++i) {
            const int tl = 2 * (i * kGW + wave) + hlf;
            const int64_t t = t0 + tl;
            const int n = f0 + 8 * l32;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + tl * 512 + 16 * (l32 ^ (tl & 31)));
            if (t < p.T && n < p.N) st16(p.out + t * p.ld_out + n, v);
        }
    } else {
        static_assert(BT == 256, "the out projection runs whole tiles");
        // Rows i kGW + wave of each half, lane = 4 consecutive features.  The
        // residual and gate values of the first half are loaded before the
        // staging; each register is reloaded for the second half as soon as
        // the first half has used it, so the load latency overlaps the work.
        constexpr int kRows = 128 / kGW;
        const int n = f0 + 4 * lane;
        u32x2_t xr[kRows], gr[kRows];
        int32_t mr[kRows];
        // the rows' adaLN table entries first (one value per wavefront), so
        // no residual or gate load waits behind another one's
        // (loaded unconditionally at a clamped row, masked where used, so
        // the loads are all in flight together)
        auto load_mod = [&](int half) {
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int64_t t = t0 + 128 * half + i * kGW + wave;
                mr[i] = p.mod_row[t < p.T ? t : p.T - 1];
            }
        };
        auto load_rows = [&](int half, int i) {
            const int64_t t = t0 + 128 * half + i * kGW + wave;
            const int64_t m = t < p.T ? mr[i] : -1;
            xr[i] = u32x2_t{0u, 0u};
            gr[i] = u32x2_t{0u, 0u};
            if (t < p.T && n < p.N) xr[i] = *reinterpret_cast<const u32x2_t*>(p.resid + t * int64_t(p.N) + n);
            if (m >= 0 && m < p.n_rows && n < p.N)
                gr[i] = *reinterpret_cast<const u32x2_t*>(p.gate + m * int64_t(p.N) + n);
        };
        load_mod(0);
#pragma unroll
        for (int i = 0; i < kRows; ++i) load_rows(0, i);
        load_mod(1);
        lds_barrier();                     // every wavefront is done with the stages
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) lds_barrier();      // every wavefront is done reading the first half
            if (wt == half) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int row = 32 * tb + l32;
#pragma unroll
                    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int c = 16 * wf + 8 * fb + 2 * g + hlf;   // 4-feature chunk of the row
                            const f32x4_t v = {acc[fb][tb][4 * g], acc[fb][tb][4 * g + 1], acc[fb][tb][4 * g + 2],
                                               acc[fb][tb][4 * g + 3]};
                            *reinterpret_cast<f32x4_t*>(smem + row * 1024 + 16 * (c ^ (row & 15))) = v;
                        }
                }
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int row = i * kGW + wave;
                const int64_t t = t0 + 128 * half + row;
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(smem + row * 1024 + 16 * (lane ^ (row & 15)));
                u32x2_t val;
                val[0] = pack_bf16x2(bf_lo(xr[i][0]) + bf_lo(gr[i][0]) * v[0], bf_hi(xr[i][0]) + bf_hi(gr[i][0]) * v[1]);
                val[1] = pack_bf16x2(bf_lo(xr[i][1]) + bf_lo(gr[i][1]) * v[2], bf_hi(xr[i][1]) + bf_hi(gr[i][1]) * v[3]);
                if (t < p.T && n < p.N) *reinterpret_cast<u32x2_t*>(p.out + t * p.ld_out + n) = val;
                if (half == 0) load_rows(1, i);
            }
        }
    }
}

// One tile of BT tokens from token t0 and features 256 ft.
template <int MODE, int BT>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const int ft, const int64_t t0, unsigned char* smem) {
    using S = Tile<BT>;
    constexpr int kTB = S::kTB;
    constexpr int kDmaPerWave = S::kDmaPerWave;
    constexpr int kStageB = S::kStageB;
    const int f0 = ft * kBF;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int wf = wave & 3;      // 64-feature quarter of the tile
    const int wt = wave >> 2;     // token half of the tile

    const uint32_t kbytes = uint32_t(p.K) * 2u;
    const uint32_t abytes = uint32_t(p.ld_act) * 2u;
    const __amdgpu_buffer_rsrc_t w_rs =
        make_rsrc(p.w + int64_t(f0) * p.K, uint64_t(p.N - f0) * kbytes);
    const __amdgpu_buffer_rsrc_t a_rs =
        make_rsrc(p.act + t0 * p.ld_act, uint64_t(p.T - t0) * abytes);

    // Direct loads: instruction n of a stage fills LDS rows
    // [kRowsPerDma n, kRowsPerDma (n+1)); lane i lands in row
    // kRowsPerDma n + i / kChunks, slot i % kChunks, and so fetches the
    // global chunk (slot ^ sw(row)) of that row.  Rows below kBF are weight
    // rows, the rest activation rows.  Wavefront w issues instructions
    // w, w + kGW, ...
    uint32_t voff[kDmaPerWave];
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
        const int n = wave + kGW * j;
        const int row = kRowsPerDma * n + lane / kChunks;
        const uint32_t c16 = 16u * uint32_t((lane % kChunks) ^ swz(row));
        voff[j] = row < kBF ? uint32_t(row) * kbytes + c16 : uint32_t(row - kBF) * abytes + c16;
    }
    auto issue = [&](int s, int buf) {
        unsigned char* base = smem + buf * kStageB;
        const uint32_t soff = uint32_t(s) * kBK * 2u;
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const int n = wave + kGW * j;
            if (n < kDmaW)
                dma16(w_rs, base + 1024 * n, voff[j], soff);
            else
                dma16(a_rs, base + 1024 * n, voff[j], soff);
        }
    };

    f32x16_t acc[2][kTB];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;

    // Fragment rows: weight rows 64 wf + 32 fb + l32, activation rows
    // kBF + kWT wt + 32 tb + l32; their swizzle is sw(l32) for all of them
    // (the row offsets are multiples of 16).  K sub-step kk reads chunk
    // 2 kk + h.
    const int sw = swz(l32);
    const int a_rd = (64 * wf + l32) * kRowB;
    const int b_rd = (kBF + S::kWT * wt + l32) * kRowB;
    int cofs[kBK / 16];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) cofs[kk] = 16 * ((2 * kk + hlf) ^ sw);
    // Stage s % 2 holds step s.  The barrier of step s sits before the MFMAs
    // of its last K sub-step: past it, every wavefront has finished reading
    // stage s (so step s + 2 may refill it) and step s + 1 has landed, so the
    // first fragments of step s + 1 and the loads of step s + 2 are issued
    // while those MFMAs run.  The scheduling groups keep each sub-step's
    // fragment reads ahead of the MFMAs of the sub-step before it (two
    // fragment sets).
    const int nks = (p.K + kBK - 1) / kBK;
    constexpr int kSub = kBK / 16;
    constexpr int kReads = 2 + kTB;           // fragments per sub-step
    constexpr int kMfma = 2 * kTB;            // MFMAs per sub-step
    static_assert(kSub % 2 == 0, "fragment sets alternate within a step");
    // direct loads per MFMA after the barrier (the rest follow the last one)
    constexpr int kLoadsPerMfma = kMfma > 1 ? (kDmaPerWave + kMfma - 2) / (kMfma - 1) : kDmaPerWave;
    bf16x8_t af[2][2], bf[2][kTB];
    auto rd = [&](int buf, const unsigned char* st, int kk) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
            af[buf][fb] = *reinterpret_cast<const bf16x8_t*>(st + a_rd + 32 * fb * kRowB + cofs[kk]);
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb)
            bf[buf][tb] = *reinterpret_cast<const bf16x8_t*>(st + b_rd + 32 * tb * kRowB + cofs[kk]);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int tb = 0; tb < kTB; ++tb)
                acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][fb], bf[buf][tb], acc[fb][tb], 0, 0, 0);
    };
    auto substeps = [&](const unsigned char* st) {
#pragma unroll
        for (int kk = 0; kk + 1 < kSub; ++kk) {
            rd((kk + 1) & 1, st, kk + 1);
            mma(kk & 1);
            __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);   // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);    // MFMA
        }
    };
    // Step s.  kNext: a step s + 1 follows (barrier, its first fragments);
    // kLoad: step s + 2 exists and is loaded into stage s % 2.
    auto step = [&](int s, auto kNext, auto kLoad) {
        substeps(smem + (s & 1) * kStageB);
        if constexpr (decltype(kNext)::value) {
            // this wavefront's reads of stage s are done and its loads of
            // step s + 1 (the only ones in flight) have landed; the barrier
            // makes both hold for every wavefront
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<0>();
            __syncthreads();
            rd(0, smem + ((s + 1) & 1) * kStageB, 0);
            if constexpr (decltype(kLoad)::value) issue(s + 2, s & 1);
            mma((kSub - 1) & 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);   // DS reads
            if constexpr (decltype(kLoad)::value) {
#pragma unroll
                for (int i = 0; i + 1 < kMfma; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerMfma, 0);   // direct loads
                }
                if constexpr (kMfma == 1) __builtin_amdgcn_sched_group_barrier(0x020, kDmaPerWave, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, kMfma - 1, 0);
            }
        } else {
            mma((kSub - 1) & 1);
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    issue(0, 0);
    if (nks > 1) {
        issue(1, 1);
        wait_vm<kDmaPerWave>();
    } else {
        wait_vm<0>();
    }
    __syncthreads();   // step 0 has landed for every wavefront
    rd(0, smem, 0);
    int s = 0;
    for (; s + 2 < nks; ++s) step(s, yes{}, yes{});
    if (s + 1 < nks) step(s++, yes{}, no{});
    step(s, no{}, no{});

    gemm_epilogue<MODE, BT>(p, acc, f0, t0, smem);
}

template <int MODE>
__global__ __launch_bounds__(kGT) void gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int b = blockIdx.x;
    int ft, tt;
    if (b < p.n_full) {
        // whole tiles first, in the XCD-contiguous order
        tile_of(p, xcd_order(b, p.n_full), ft, tt);
        gemm_tile<MODE, kBT>(p, ft, int64_t(tt) * kBT, smem);
        return;
    }
    if constexpr (MODE == kModeQkv) {
        // then the last round's tiles, each cut into p.slices token slices
        // (the dispatcher starts these last, as whole tiles free their CUs)
        const int li = xcd_order(b - p.n_full, int(gridDim.x) - p.n_full);
        const int part = li % p.slices;
        tile_of(p, p.n_full + li / p.slices, ft, tt);
        const int64_t t0 = int64_t(tt) * kBT + int64_t(part) * (kBT / p.slices);
        if (t0 >= p.T) return;   // a slice past the last token (every wavefront leaves together)
        if (p.slices == 4)
            gemm_tile<MODE, kBT / 4>(p, ft, t0, smem);
        else
            gemm_tile<MODE, kBT / 2>(p, ft, t0, smem);
    }
}

// ---------------------------------------------------------------------------
// adaLN of the residual stream: u = LN(x) * (1 + scale[m]) + shift[m], bf16
// ---------------------------------------------------------------------------
constexpr int kLnTokensPerBlock = 4;

// The same wavefront also writes the token's row of the rotation table.
template <int NCH>
__global__ __launch_bounds__(256) void adaln_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                    const uint16_t* __restrict__ shift,
                                                    const uint16_t* __restrict__ scale,
                                                    const int32_t* __restrict__ mod_row, int n_rows,
                                                    uint16_t* __restrict__ u, int64_t T, int C, float eps,
                                                    RopeTableParams rp) {
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * kLnTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    rope_table_row(rp, t, lane);
    const int nch = C >> 3;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(x + t * ld_x, row_bytes);
    u32x4_t px[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) px[i] = bload16(x_rs, 16u * uint32_t(lane + kWave * i), 0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) s += bf_lo(px[i][w]) + bf_hi(px[i][w]);
    const float invC = 1.0f / float(C);
    const float mean = wave_sum(s) * invC;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const bool in = lane + kWave * i < nch;   // zero-filled chunks are not row data
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a0 = bf_lo(px[i][w]) - mean, a1 = bf_hi(px[i][w]) - mean;
            v += in ? a0 * a0 + a1 * a1 : 0.f;
        }
    }
    const float rstd = rsqrtf(wave_sum(v) * invC + eps);
    // a row outside [0, n_rows) gets empty resources: its loads read zeros
    const int64_t m = __builtin_amdgcn_readfirstlane(mod_row[t]);
    const bool mok = m >= 0 && m < n_rows;
    const __amdgpu_buffer_rsrc_t sh_rs = make_rsrc(shift + (mok ? m : 0) * C, mok ? row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(scale + (mok ? m : 0) * C, mok ? row_bytes : 0u);
    const __amdgpu_buffer_rsrc_t u_rs = make_rsrc(u + t * C, row_bytes);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const uint32_t off = 16u * uint32_t(lane + kWave * i);
        float fx[8], fs[8], fc[8], r[8];
        unpack8(px[i], fx);
        unpack8(bload16(sh_rs, off, 0), fs);
        unpack8(bload16(sc_rs, off, 0), fc);
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (fx[j] - mean) * rstd * (1.0f + fc[j]) + fs[j];
        bstore16(u_rs, off, 0, pack8(r));
    }
}

// The rotation table alone (no modulation pass to carry it): one wavefront
// per token.
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableParams rp, int64_t T) {
    const int64_t t = int64_t(blockIdx.x) * kLnTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    rope_table_row(rp, t, threadIdx.x & 63);
}

template <int NCH>
hipError_t launch_adaln_nch(const BlockQkvArgs& a, uint16_t* u, const RopeTableParams& rp, hipStream_t stream) {
    const int64_t blocks = (a.T + kLnTokensPerBlock - 1) / kLnTokensPerBlock;
    hipLaunchKernelGGL(adaln_kernel<NCH>, dim3(unsigned(blocks)), dim3(256), 0, stream, a.x, a.ld_x, a.shift,
                       a.scale, a.mod_row, a.n_rows, u, a.T, a.H * a.D, a.eps, rp);
    return hipGetLastError();
}

hipError_t launch_adaln(const BlockQkvArgs& a, uint16_t* u, const RopeTableParams& rp, hipStream_t stream) {
    const int per_lane = (a.H * a.D / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) return launch_adaln_nch<1>(a, u, rp, stream);
    if (per_lane <= 2) return launch_adaln_nch<2>(a, u, rp, stream);
    if (per_lane <= 4) return launch_adaln_nch<4>(a, u, rp, stream);
    if (per_lane <= 6) return launch_adaln_nch<6>(a, u, rp, stream);
    if (per_lane <= 8) return launch_adaln_nch<8>(a, u, rp, stream);
    if (per_lane <= 12) return launch_adaln_nch<12>(a, u, rp, stream);
    return launch_adaln_nch<16>(a, u, rp, stream);
}

// Whole tiles run in rounds of `cus` (one workgroup per CU).  For the QKV
// projection a last round at most half full is cut into token slices of the
// same 256 features: two of 128 tokens, or four of 64 when that still fits
// the CUs, so the round takes a half or a quarter of a tile's time with the
// full K in each workgroup (no partial sums to add).
struct TailPlan {
    int n_full, slices;
};
TailPlan tail_plan(int n_tiles, int cus) {
    TailPlan tp{n_tiles, 1};
    if (cus <= 0) return tp;
    const int tail = n_tiles % cus;
    if (tail == 0 || 2 * tail > cus) return tp;
    tp.n_full = n_tiles - tail;
    tp.slices = 4 * tail <= cus ? 4 : 2;
    return tp;
}

// Bytes of the modulated rows and of the rotation table (each 256-byte
// aligned).
size_t qkv_rows_bytes(int64_t T, int C) { return (size_t(T) * size_t(C) * 2 + 255) & ~size_t(255); }
size_t qkv_table_bytes(int64_t T, int D) { return (size_t(T) * size_t(D) * 4 + 255) & ~size_t(255); }

template <int MODE>
hipError_t launch_gemm(GemmParams& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MODE>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsB);
    if (attr != hipSuccess) return attr;
    p.tiles_f = (p.N + kBF - 1) / kBF;
    p.tiles_t = int((p.T + kBT - 1) / kBT);
    const int n_tiles = p.tiles_f * p.tiles_t;
    p.n_full = n_tiles;
    p.slices = 1;
    if (MODE == kModeQkv) {
        const TailPlan tp = tail_plan(n_tiles, device_cu_count());
        p.n_full = tp.n_full;
        p.slices = tp.slices;
    }
    const int grid = p.n_full + (n_tiles - p.n_full) * p.slices;
    hipLaunchKernelGGL(gemm_kernel<MODE>, dim3(unsigned(grid)), dim3(kGT), kLdsB, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t block_qkv_workspace_bytes(int64_t T, int32_t C, int32_t D) {
    if (T <= 0 || C <= 0 || D <= 0) return 0;
    return qkv_rows_bytes(T, C) + qkv_table_bytes(T, D);
}

hipError_t launch_block_qkv(const BlockQkvArgs& args, hipStream_t stream) {
    if (args.T == 0) return hipSuccess;
    const int C = args.H * args.D;
    unsigned char* ws = static_cast<unsigned char*>(args.workspace);
    // workspace: modulated rows, rotation table
    RopeTableParams rp = {};
    rp.cs = reinterpret_cast<f32x2_t*>(ws + qkv_rows_bytes(args.T, C));
    rp.pos = args.pos;
    rp.D = args.D;
    rp.rope_f = args.rope_f;
    rp.rope_r = args.rope_r;
    const int dims[3] = {args.rope_f, args.rope_r, args.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            rp.theta_turns[pair++] = std::pow(double(args.rope_base), -2.0 * j / double(dims[ax])) *
                                     0.15915494309189535;   // radians -> turns (1 / 2 pi)
    const uint16_t* act = args.x;
    int64_t ld_act = args.ld_x;
    if (args.shift != nullptr) {
        uint16_t* u = reinterpret_cast<uint16_t*>(ws);   // the modulated rows
        const hipError_t e = launch_adaln(args, u, rp, stream);
        if (e != hipSuccess) return e;
        act = u;
        ld_act = C;
    } else {
        const int64_t blocks = (args.T + kLnTokensPerBlock - 1) / kLnTokensPerBlock;
        hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, rp, args.T);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    GemmParams p = {};
    p.w = args.w;
    p.act = act;
    p.ld_act = ld_act;
    p.T = args.T;
    p.N = 3 * C;
    p.K = C;
    p.out = args.qkv;
    p.ld_out = args.ld_qkv;
    p.rope_limit = 2 * C;
    p.D = args.D;
    p.rope_cs = rp.cs;
    return launch_gemm<kModeQkv>(p, stream);
}

hipError_t launch_block_out(const BlockOutArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    GemmParams p = {};
    p.w = a.w;
    p.act = a.o;
    p.ld_act = a.ld_o;
    p.T = a.T;
    p.N = a.C;
    p.K = a.C;
    p.out = a.y;
    p.ld_out = a.C;
    p.resid = a.x;
    p.gate = a.gate;
    p.mod_row = a.mod_row;
    p.n_rows = a.n_rows;
    return launch_gemm<kModeOut>(p, stream);
}

}  // namespace mf
