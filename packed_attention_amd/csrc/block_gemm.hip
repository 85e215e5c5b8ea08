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
//    through two LDS stages filled by direct global->LDS loads one step
//    ahead (no staging registers); LDS rows are 128 bytes with their 16-byte
//    chunks swizzled, so the fragment reads are conflict-free without
//    padding.
//    Transposed output: each lane holds one token and 16 features, so the
//    RoPE pairs (adjacent features) sit in one lane and each lane stores 4
//    consecutive features (8 bytes) per register group.
//  * Tiles are numbered so that the tiles one XCD runs are consecutive and
//    share their weight tile (its L2 serves the re-reads).
//  * Split tail (QKV projection): one workgroup per CU, so the tiles run in
//    rounds of #CUs; when the last round is less than half full, each of its
//    tiles is cut into s K-ranges (s = #CUs / tail tiles) that run side by
//    side and write fp32 partial tiles to the workspace, and
//    gemm_fixup_kernel adds the pieces in a fixed order and runs the same
//    epilogue.
//  * Ragged edges: buffer resources end at the last token / feature, so rows
//    past them read as zeros; the epilogue stores only rows inside.
#include <algorithm>
#include <cmath>

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
constexpr int kStageRows = kBF + kBT;
constexpr int kStageB = kStageRows * kRowB;
constexpr int kStages = 2;
constexpr int kLdsB = kStages * kStageB;   // 128 KiB
static_assert(kStages >= 2 && kStages <= 4, "waits below cover up to two later groups");
constexpr int kRowsPerDma = 64 / kChunks;  // LDS rows one direct-load instruction fills
constexpr int kDma = kStageRows / kRowsPerDma;   // direct-load instructions per stage
constexpr int kDmaW = kBF / kRowsPerDma;         // of which fill the weight rows
constexpr int kDmaPerWave = kDma / kGW;
constexpr int kXcds = 8;
constexpr int kGroupF = 4;                 // feature tiles per group of the tile order
static_assert(kDma % kGW == 0, "whole direct-load instructions");
// The epilogue stages the bf16 output tile [kBT tokens][kBF features]
// through the (then free) LDS stages.
static_assert(kBT * kBF * 2 <= kLdsB, "output tile fits the LDS stages");

// LDS rows are stored swizzled: chunk c of row r sits in slot c ^ sw(r),
// sw(r) = (r / 2) % 8.  The 16 lanes one LDS cycle serves read 16-byte
// chunks of 16 consecutive rows (two per 256-byte bank line), and the swizzle
// gives each of them its own 4 banks without padding.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

enum { kModeQkv = 0, kModeOut = 1 };

struct GemmParams {
    const uint16_t* w;       // [N][K]
    const uint16_t* act;     // [T][K], token stride ld_act
    int64_t ld_act;
    int64_t T;
    int N, K;
    uint16_t* out;           // [T][N], token stride ld_out
    int64_t ld_out;
    // QKV: RoPE on the features below rope_limit (q and k)
    int rope_limit, D, rope_f, rope_r;
    const int32_t* pos;
    // out projection: y = resid + gate[m] * acc
    const uint16_t* resid;
    const uint16_t* gate;
    const int32_t* mod_row;
    int tiles_t, tiles_f;
    // split tail: tiles [n_full, tiles) run as `split` K-ranges each, fp32
    // partial tiles in `partial` (kTileAcc floats per piece)
    int n_full, split;
    float* partial;
    double theta_turns[64];
};

constexpr int kTileAcc = kBF * kBT;        // fp32 accumulators of one tile

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
// of block fb = feature 8(r/4) + 4h + r%4 of the block).  The finished bf16
// values go to an LDS image of the output tile (rows = tokens, 512 bytes;
// 16-byte chunk c of row t in slot c ^ (t % 32), so the 8-byte writes of 32
// consecutive rows and the 16-byte reads along a row are both
// conflict-free), then out to global memory one 512-byte row segment per 32
// lanes.
template <int MODE>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, f32x16_t (&acc)[2][4], const int f0,
                                              const int64_t t0, unsigned char* smem) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int wf = wave & 3;
    const int wt = wave >> 2;
    __syncthreads();                       // every wavefront is done with the stages
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int tl = 128 * wt + 32 * tb + l32;   // token row inside the tile
        const int64_t t = t0 + tl;
        int64_t m = 0;
        if constexpr (MODE == kModeOut) m = t < p.T ? p.mod_row[t] : 0;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
            const int fl = 64 * wf + 32 * fb;      // first feature of the block inside the tile
            const int nblk = f0 + fl;
            f32x16_t& a = acc[fb][tb];
            if constexpr (MODE == kModeQkv) {
                if (nblk < p.rope_limit && t < p.T) {
                    // q or k: turn each adjacent pair (r, r+1) by pos_axis *
                    // theta; the angle is formed in fp64 in turns and reduced
                    // to [-1/2, 1/2] before the hardware sine and cosine
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const int e = (nblk + 8 * (r >> 2) + 4 * hlf + (r & 3)) % p.D;
                        const int axis = e < p.rope_f ? 0 : (e < p.rope_f + p.rope_r ? 1 : 2);
                        const double turns = double(p.pos[3 * t + axis]) * p.theta_turns[e >> 1];
                        const float f = float(turns - rint(turns));
                        const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
                        const float x0 = a[r], x1 = a[r + 1];
                        a[r] = x0 * cs - x1 * sn;
                        a[r + 1] = x0 * sn + x1 * cs;
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int f = fl + 8 * g + 4 * hlf;        // feature inside the tile
                float v0 = a[4 * g], v1 = a[4 * g + 1], v2 = a[4 * g + 2], v3 = a[4 * g + 3];
                if constexpr (MODE == kModeOut) {
                    if (t < p.T && f0 + f < p.N) {
                        const int64_t n0 = f0 + f;
                        const u32x2_t xr = *reinterpret_cast<const u32x2_t*>(p.resid + t * int64_t(p.N) + n0);
                        const u32x2_t gr = *reinterpret_cast<const u32x2_t*>(p.gate + m * int64_t(p.N) + n0);
                        v0 = bf_lo(xr[0]) + bf_lo(gr[0]) * v0;
                        v1 = bf_hi(xr[0]) + bf_hi(gr[0]) * v1;
                        v2 = bf_lo(xr[1]) + bf_lo(gr[1]) * v2;
                        v3 = bf_hi(xr[1]) + bf_hi(gr[1]) * v3;
                    }
                }
                u32x2_t val;
                val[0] = pack_bf16x2(v0, v1);
                val[1] = pack_bf16x2(v2, v3);
                const int slot = (f >> 3) ^ (tl & 31);
                *reinterpret_cast<u32x2_t*>(smem + tl * 512 + 16 * slot + 8 * ((f >> 2) & 1)) = val;
            }
        }
    }
    __syncthreads();
    // rows 2 (i kGW + wave) + h, chunk l32: 32 lanes per 512-byte row segment
#pragma unroll 4
    for (int i = 0; i < kBT / (2 * kGW); ++i) {
        const int tl = 2 * (i * kGW + wave) + hlf;
        const int64_t t = t0 + tl;
        const int n = f0 + 8 * l32;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + tl * 512 + 16 * (l32 ^ (tl & 31)));
        if (t < p.T && n < p.N) st16(p.out + t * p.ld_out + n, v);
    }
}

template <int MODE>
__global__ __launch_bounds__(kGT) void gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int b = blockIdx.x;
    // whole tiles first (blockIdx < n_full), then the pieces of the split
    // tail tiles, which the dispatcher starts last
    const bool piece = b >= p.n_full;
    int lt, part = 0;
    if (!piece) {
        lt = xcd_order(b, p.n_full);
    } else {
        const int li = xcd_order(b - p.n_full, int(gridDim.x) - p.n_full);
        lt = p.n_full + li / p.split;
        part = li - (li / p.split) * p.split;
    }
    int ft, tt;
    tile_of(p, lt, ft, tt);
    const int f0 = ft * kBF;
    const int64_t t0 = int64_t(tt) * kBT;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int wf = wave & 3;      // 64-feature quarter of the tile
    const int wt = wave >> 2;     // 128-token half of the tile

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

    f32x16_t acc[2][4];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fb][tb][r] = 0.f;

    // Fragment rows: weight rows 64 wf + 32 fb + l32, activation rows
    // kBF + 128 wt + 32 tb + l32; their swizzle is sw(l32) for all of them
    // (the row offsets are multiples of 16).  K sub-step kk reads chunk
    // 2 kk + h.
    const int sw = swz(l32);
    const int a_rd = (64 * wf + l32) * kRowB;
    const int b_rd = (kBF + 128 * wt + l32) * kRowB;
    int cofs[kBK / 16];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) cofs[kk] = 16 * ((2 * kk + hlf) ^ sw);
    // K steps [ks0, ks1): all of them, or this piece's share
    const int nks_all = (p.K + kBK - 1) / kBK;
    const int ks0 = piece ? part * nks_all / p.split : 0;
    const int ks1 = piece ? (part + 1) * nks_all / p.split : nks_all;
    const int nks = ks1 - ks0;
    constexpr int kAhead = kStages - 1;        // steps loaded ahead
    for (int s = 0; s < kAhead; ++s)
        if (s < nks) issue(ks0 + s, s % kStages);
    for (int s = 0; s < nks; ++s) {
        // this wavefront's loads of stage s have landed once at most the
        // later groups (up to kAhead - 1 of them) are still in flight
        const int later = min(kAhead - 1, nks - 1 - s);
        if constexpr (kAhead >= 3) {
            if (later >= 2) wait_vm<2 * kDmaPerWave>();
        }
        if constexpr (kAhead >= 2) {
            if (later == 1) wait_vm<kDmaPerWave>();
        }
        if (later == 0) wait_vm<0>();
        // stage s landed for every wavefront; the stage refilled next was
        // last read in step s-1, which every wavefront has finished
        __syncthreads();
        if (s + kAhead < nks) issue(ks0 + s + kAhead, (s + kAhead) % kStages);
        const unsigned char* st = smem + (s % kStages) * kStageB;
        // K sub-steps: the six fragments of sub-step kk+1 are read while
        // the eight MFMAs of sub-step kk run
        bf16x8_t af[2][2], bf[2][4];
        auto rd = [&](int buf, int kk) {
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
                af[buf][fb] = *reinterpret_cast<const bf16x8_t*>(st + a_rd + 32 * fb * kRowB + cofs[kk]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                bf[buf][tb] = *reinterpret_cast<const bf16x8_t*>(st + b_rd + 32 * tb * kRowB + cofs[kk]);
        };
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            if (kk + 1 < kBK / 16) rd((kk + 1) & 1, kk + 1);
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][fb], bf[kk & 1][tb],
                                                                          acc[fb][tb], 0, 0, 0);
        }
    }

    if (piece) {
        // fp32 partial tile in fragment order: 16-byte groups of four
        // registers, 64 lanes side by side (1 KiB per store instruction)
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(p.partial + size_t((lt - p.n_full) * p.split + part) * kTileAcc);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4_t v = {acc[fb][tb][4 * g], acc[fb][tb][4 * g + 1], acc[fb][tb][4 * g + 2],
                                       acc[fb][tb][4 * g + 3]};
                    dst[(((wave * 2 + fb) * 4 + tb) * 4 + g) * 64 + lane] = v;
                }
        return;
    }
    gemm_epilogue<MODE>(p, acc, f0, t0, smem);
}

// Sum of the pieces of split tail tile n_full + blockIdx.x (in piece order),
// then the same epilogue as a whole tile.
template <int MODE>
__global__ __launch_bounds__(kGT) void gemm_fixup_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int lt = p.n_full + int(blockIdx.x);
    int ft, tt;
    tile_of(p, lt, ft, tt);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    f32x16_t acc[2][4];
    for (int part = 0; part < p.split; ++part) {
        const f32x4_t* src =
            reinterpret_cast<const f32x4_t*>(p.partial + size_t((lt - p.n_full) * p.split + part) * kTileAcc);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4_t v = src[(((wave * 2 + fb) * 4 + tb) * 4 + g) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[fb][tb][4 * g + e] = part == 0 ? v[e] : acc[fb][tb][4 * g + e] + v[e];
                }
    }
    gemm_epilogue<MODE>(p, acc, ft * kBF, int64_t(tt) * kBT, smem);
}

// ---------------------------------------------------------------------------
// adaLN of the residual stream: u = LN(x) * (1 + scale[m]) + shift[m], bf16
// ---------------------------------------------------------------------------
constexpr int kLnTokensPerBlock = 4;

template <int NCH>
__global__ __launch_bounds__(256) void adaln_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                    const uint16_t* __restrict__ shift,
                                                    const uint16_t* __restrict__ scale,
                                                    const int32_t* __restrict__ mod_row,
                                                    uint16_t* __restrict__ u, int64_t T, int C, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t t = int64_t(blockIdx.x) * kLnTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
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
    const int64_t m = __builtin_amdgcn_readfirstlane(mod_row[t]);
    const __amdgpu_buffer_rsrc_t sh_rs = make_rsrc(shift + m * C, row_bytes);
    const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(scale + m * C, row_bytes);
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

template <int NCH>
hipError_t launch_adaln_nch(const BlockQkvArgs& a, uint16_t* u, hipStream_t stream) {
    const int64_t blocks = (a.T + kLnTokensPerBlock - 1) / kLnTokensPerBlock;
    hipLaunchKernelGGL(adaln_kernel<NCH>, dim3(unsigned(blocks)), dim3(256), 0, stream, a.x, a.ld_x, a.shift,
                       a.scale, a.mod_row, u, a.T, a.H * a.D, a.eps);
    return hipGetLastError();
}

hipError_t launch_adaln(const BlockQkvArgs& a, uint16_t* u, hipStream_t stream) {
    const int per_lane = (a.H * a.D / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) return launch_adaln_nch<1>(a, u, stream);
    if (per_lane <= 2) return launch_adaln_nch<2>(a, u, stream);
    if (per_lane <= 4) return launch_adaln_nch<4>(a, u, stream);
    if (per_lane <= 6) return launch_adaln_nch<6>(a, u, stream);
    if (per_lane <= 8) return launch_adaln_nch<8>(a, u, stream);
    if (per_lane <= 12) return launch_adaln_nch<12>(a, u, stream);
    return launch_adaln_nch<16>(a, u, stream);
}

// Whole tiles run in rounds of `cus` (one workgroup per CU); a last round
// under half full is cut into K-ranges of at least four steps.
struct SplitPlan {
    int n_full, split;
};
SplitPlan split_plan(int n_tiles, int nks, int cus) {
    SplitPlan sp{n_tiles, 1};
    if (cus <= 0) return sp;
    const int tail = n_tiles % cus;
    if (tail == 0) return sp;
    const int s = std::min(cus / tail, nks / 4);
    if (s < 2) return sp;
    sp.n_full = n_tiles - tail;
    sp.split = s;
    return sp;
}

int qkv_tiles(int64_t T, int C) { return ((3 * C + kBF - 1) / kBF) * int((T + kBT - 1) / kBT); }

// Bytes of the modulated rows (256-byte aligned) and of the partial tiles.
size_t qkv_rows_bytes(int64_t T, int C) { return (size_t(T) * size_t(C) * 2 + 255) & ~size_t(255); }
size_t qkv_partial_bytes(int64_t T, int C, int cus) {
    const int tiles = qkv_tiles(T, C);
    const SplitPlan sp = split_plan(tiles, (C + kBK - 1) / kBK, cus);
    return sp.split > 1 ? size_t(tiles - sp.n_full) * sp.split * kTileAcc * sizeof(float) : 0;
}

template <int MODE>
hipError_t launch_gemm(GemmParams& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MODE>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsB);
    if (attr != hipSuccess) return attr;
    p.tiles_f = (p.N + kBF - 1) / kBF;
    p.tiles_t = int((p.T + kBT - 1) / kBT);
    const int n_tiles = p.tiles_f * p.tiles_t;
    p.n_full = n_tiles;
    p.split = 1;
    if (p.partial != nullptr) {
        const SplitPlan sp = split_plan(n_tiles, (p.K + kBK - 1) / kBK, device_cu_count());
        p.n_full = sp.n_full;
        p.split = sp.split;
    }
    const int grid = p.n_full + (n_tiles - p.n_full) * p.split;
    hipLaunchKernelGGL(gemm_kernel<MODE>, dim3(unsigned(grid)), dim3(kGT), kLdsB, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split == 1) return e;
    static const hipError_t attr_fix = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_fixup_kernel<MODE>), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsB);
    if (attr_fix != hipSuccess) return attr_fix;
    hipLaunchKernelGGL(gemm_fixup_kernel<MODE>, dim3(unsigned(n_tiles - p.n_full)), dim3(kGT), kLdsB, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t block_qkv_workspace_bytes(int64_t T, int32_t C) {
    if (T <= 0 || C <= 0) return 0;
    int cus = device_cu_count();
    if (cus <= 0) cus = 256;   // no device visible: size for an MI355X
    return qkv_rows_bytes(T, C) + qkv_partial_bytes(T, C, cus);
}

hipError_t launch_block_qkv(const BlockQkvArgs& args, hipStream_t stream) {
    if (args.T == 0) return hipSuccess;
    const int C = args.H * args.D;
    const uint16_t* act = args.x;
    int64_t ld_act = args.ld_x;
    if (args.shift != nullptr) {
        uint16_t* u = static_cast<uint16_t*>(args.workspace);   // the modulated rows
        const hipError_t e = launch_adaln(args, u, stream);
        if (e != hipSuccess) return e;
        act = u;
        ld_act = C;
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
    p.rope_f = args.rope_f;
    p.rope_r = args.rope_r;
    p.pos = args.pos;
    // the split tail's partial tiles follow the modulated rows
    p.partial = reinterpret_cast<float*>(static_cast<unsigned char*>(args.workspace) + qkv_rows_bytes(args.T, C));
    const int dims[3] = {args.rope_f, args.rope_r, args.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            p.theta_turns[pair++] = std::pow(double(args.rope_base), -2.0 * j / double(dims[ax])) *
                                    0.15915494309189535;   // radians -> turns (1 / 2 pi)
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
    return launch_gemm<kModeOut>(p, stream);
}

}  // namespace mf
