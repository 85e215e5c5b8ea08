// Block-diagonal (varlen) softmax attention backward for gfx950.
//
// What it computes: the gradients dQ, dK, dV of O = softmax(tau Q K^T) V,
// per packed sequence and head, given dO and the forward's row log-sum-exp.
// With P = softmax rows and D_i = sum_e dO[i,e] O[i,e]:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = tau dS K,
//   dK = tau dS^T Q.
// P is recomputed from the forward's LSE: P = exp(tau S - LSE) (exact, no
// running max).  Sources: the method's attention is the block-diagonal joint
// attention of the picx.dev summary of Mage-Flow, Methodology >
// Native-Resolution MMDiT (variable-length kernels over packed samples with
// per-sample cumulative offsets); the pages report training with these
// kernels (Methodology > Training Infrastructure), whose backward is this
// chain rule.
//
// Design (MI355X, CDNA4): three kernels, no atomics, deterministic.
//  * bwd_tiles_kernel: per-sequence tile counts and their prefix sums (one
//    workgroup), so work units map to (sequence, head, tile) by a binary
//    search, with no empty workgroups for packs of many short sequences.
//  * bwd_dot_kernel: D = rowsum(dO * O) in fp32, HBM-bound.
//  * attn_bwd_dkdv_kernel: a work unit is 128 keys of one head (4
//    wavefronts, one per SIMD, 32 keys each, up to 512 registers).  A
//    wavefront keeps its K and V rows in registers as MFMA B operands and
//    streams the sequence's queries in steps of 64 through LDS (Q and dO
//    tiles plus LSE and D, staged through registers one step ahead, two
//    buffers).  Per 32-query block: S = Q K^T and dP = dO V^T
//    (v_mfma_f32_32x32x16_bf16; every lane then holds one key and 16
//    queries), P and dS in fp32 VALU, then dV^T += dO^T P and dK^T += Q^T dS
//    with dO^T / Q^T read transposed from LDS (ds_read_b64_tr_b16) and P / dS
//    rounded to bf16 straight from the accumulator layout as the B operand.
//    A step is one compile-time sequence of 64 MFMAs with every LDS operand
//    read six MFMAs ahead and each block's VALU work threaded through the
//    other block's MFMAs (with one wavefront per SIMD nothing else hides LDS
//    latency or VALU time).  The accumulators are transposed (d x keys), so
//    the epilogue stores 4 consecutive dims per lane.
//  * attn_bwd_dq_kernel: a work unit is 256 queries of one head (8
//    wavefronts, 2 per SIMD, 32 queries each), the forward's structure: Q and
//    dO rows in registers, K and V tiles of 64 keys through LDS,
//    S^T = K Q^T and dP^T = V dO^T (every lane holds one query and 16 keys,
//    so LSE and D are per-lane scalars), dS^T in VALU, dQ^T += K^T dS^T with
//    K^T read transposed.
//  * Rows that are read both row-wise (16-byte reads) and transposed are
//    padded to 2D+48 bytes: the 16-byte reads are conflict-free, the
//    transposed reads 2-way.  Rows read row-wise only are padded to 2D+16.
//  * Ragged tiles: buffer resources end at the sequence's last row, so rows
//    past it read as zeros.  Zero Q and dO rows contribute nothing to dK and
//    dV; keys past the end of the last key tile of the dQ kernel get P = 0.
#include <cmath>
#include <mutex>
#include <utility>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kKvWaves = 4;                // dK/dV kernel: one wavefront per SIMD
constexpr int kKvKeys = 32 * kKvWaves;     // keys per dK/dV work unit
constexpr int kKvQ = 64;                   // queries per dK/dV step
constexpr int kQWaves = 8;                 // dQ kernel: two wavefronts per SIMD
constexpr int kQRows = 32 * kQWaves;       // queries per dQ work unit
constexpr int kQK = 64;                    // keys per dQ step
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BT {
    static constexpr int KK = D / 16;              // MFMA k-steps along d
    static constexpr int EB = D / 32;              // 32-wide blocks of d
    static constexpr int KCH = D / 8;              // 16-byte chunks per row
    static constexpr int X_UNITS = KCH + 3;        // row read both ways
    static constexpr int X_ROW = 16 * X_UNITS;
    static constexpr int R_UNITS = KCH + 1;        // row read row-wise only
    static constexpr int R_ROW = 16 * R_UNITS;
    // dK/dV step: Q tile, dO tile, then LSE[64] and D[64] (fp32)
    static constexpr int QT_BYTES = kKvQ * X_ROW;
    static constexpr int KV_STAGE = 2 * QT_BYTES + 2 * kKvQ * 4;
    static constexpr int KV_LDS = 2 * KV_STAGE;                 // double-buffered
    // dQ step: K tile (read both ways), V tile (row-wise)
    static constexpr int KT_BYTES = kQK * X_ROW;
    static constexpr int VT_BYTES = kQK * R_ROW;
    static constexpr int Q_STAGE = KT_BYTES + VT_BYTES;
    static constexpr int Q_LDS = 2 * Q_STAGE;                   // double-buffered
    static_assert(kKvQ * KCH % (64 * kKvWaves) == 0, "whole staging chunks per thread");
    static_assert(kQK * KCH % (64 * kQWaves) == 0, "whole staging chunks per thread");
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;        // [H][T]
    float* dsum;             // workspace: D = rowsum(dO * O), [H][T]
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const int32_t* cu;
    const int64_t* pre_kv;   // workspace: prefix sums of key tiles per sequence [n+1]
    const int64_t* pre_q;    // workspace: prefix sums of query tiles per sequence [n+1]
    int n_seq;
    int H;
    int64_t T;
    int64_t ld_qkv, ld_o, ld_d;
    float scale;             // tau
    float c;                 // tau * log2(e)
};

// Workspace layout: D values, then the two prefix arrays, each 256-aligned.
__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }
__host__ __device__ constexpr size_t ws_dsum_bytes(int64_t T, int H) { return align256(size_t(T) * H * 4); }
__host__ __device__ constexpr size_t ws_pre_bytes(int n) { return align256(size_t(n + 1) * 8); }

// ---------------------------------------------------------------------------
// Tile prefix sums (one workgroup of 256 threads, each a contiguous chunk).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_tiles_kernel(const int32_t* __restrict__ cu, int n,
                                                        int64_t* __restrict__ pre_kv,
                                                        int64_t* __restrict__ pre_q) {
    __shared__ int64_t part_kv[256], part_q[256];
    const int tid = threadIdx.x;
    const int per = (n + 255) / 256;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    int64_t akv = 0, aq = 0;
    for (int s = s0; s < s1; ++s) {
        const int L = cu[s + 1] - cu[s];
        akv += (L + kKvKeys - 1) / kKvKeys;
        aq += (L + kQRows - 1) / kQRows;
    }
    part_kv[tid] = akv;
    part_q[tid] = aq;
    __syncthreads();
    if (tid == 0) {
        int64_t rk = 0, rq = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t a = part_kv[i], b = part_q[i];
            part_kv[i] = rk;
            part_q[i] = rq;
            rk += a;
            rq += b;
        }
        pre_kv[n] = rk;
        pre_q[n] = rq;
    }
    __syncthreads();
    int64_t bkv = part_kv[tid], bq = part_q[tid];
    for (int s = s0; s < s1; ++s) {
        pre_kv[s] = bkv;
        pre_q[s] = bq;
        const int L = cu[s + 1] - cu[s];
        bkv += (L + kKvKeys - 1) / kKvKeys;
        bq += (L + kQRows - 1) / kQRows;
    }
}

// Work unit -> (sequence, head, tile).  Units of sequence s are
// [pre[s] * H, pre[s+1] * H), head-major.  False past the last unit.
__device__ bool locate_unit(const int64_t* pre, int n, int H, int64_t unit, int& s, int& h, int& tile) {
    if (unit >= pre[n] * H) return false;
    int lo = 0, hi = n - 1;              // last s with pre[s] * H <= unit
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

// ---------------------------------------------------------------------------
// D[h][t] = sum_e dO[t,h,e] * O[t,h,e]  (fp32 from bf16)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dout, int64_t ld_o,
                                                      float* __restrict__ dsum, int64_t T, int H) {
    constexpr int TPR = D / 8;            // threads per (token, head) row, 16 bytes each
    constexpr int RPB = 256 / TPR;
    const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR;   // t * H + h
    const int part = threadIdx.x % TPR;
    const bool live = row < T * H;
    const int64_t t = live ? row / H : 0;
    const int h = live ? int(row - t * H) : 0;
    float acc = 0.f;
    if (live) {
        const u32x4_t a = ld16(o + t * ld_o + int64_t(h) * D + 8 * part);
        const u32x4_t b = ld16(dout + t * ld_o + int64_t(h) * D + 8 * part);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf_lo(a[i]) * bf_lo(b[i]) + bf_hi(a[i]) * bf_hi(b[i]);
    }
#pragma unroll
    for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (live && part == 0) dsum[int64_t(h) * T + t] = acc;
}

// Transposed 8-row x 4-dim fragment pair of a row-major tile: lanes receive
// dim 32*blk + (lane & 31) of rows {4h..4h+3} and {8+4h..8+4h+3} of the
// 16-row chunk `chunk` (h = lane / 32), as an MFMA A operand whose k index
// follows the 32x32 accumulator's row pattern.
template <int ROW>
__device__ __forceinline__ bf16x8_t tr_frag(const unsigned char* tile, int tr_rd, int chunk, int blk) {
    const unsigned char* a = tile + tr_rd + chunk * 16 * ROW + blk * 64;
    const s16x4_t lo = lds_read_tr16_b64(a);
    const s16x4_t hi = lds_read_tr16_b64(a + 8 * ROW);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Lane's byte offset for tr_frag: row (4h + (lane&15)/4) of the chunk, dims
// 16*((lane>>4)&1) + 4*(lane&3).
template <int ROW>
__device__ __forceinline__ int tr_offset(int lane) {
    return (4 * (lane >> 5) + ((lane & 15) >> 2)) * ROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

// bf16 B operand of chunk cc (16 rows of the accumulator's m index) from a
// pair of 32x32 accumulators: registers 8*(cc&1) .. +7 of block cc>>1.
__device__ __forceinline__ bf16x8_t pack_chunk(const f32x16_t& acc, int half) {
    u32x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(acc[8 * half + 2 * i], acc[8 * half + 2 * i + 1]);
    return __builtin_bit_cast(bf16x8_t, u);
}

// Store a transposed accumulator set (d x 32 rows; lane = row l32, dims
// 32m + 8gq + 4h .. +3) as bf16 rows, times `mul`.
template <int D>
__device__ __forceinline__ void store_rows_t(uint16_t* base, const f32x16_t (&acc)[D / 32], float mul, int hlf) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            u32x2_t val;
            val[0] = pack_bf16x2(acc[m][4 * gq] * mul, acc[m][4 * gq + 1] * mul);
            val[1] = pack_bf16x2(acc[m][4 * gq + 2] * mul, acc[m][4 * gq + 3] * mul);
            *reinterpret_cast<u32x2_t*>(base + 32 * m + 8 * gq + 4 * hlf) = val;
        }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(BwdParams p) {
    using TL = BT<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int seq, head, tile;
    if (!locate_unit(p.pre_kv, p.n_seq, p.H, blockIdx.x, seq, head, tile)) return;
    seq = __builtin_amdgcn_readfirstlane(seq);
    head = __builtin_amdgcn_readfirstlane(head);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int64_t tok0 = __builtin_amdgcn_readfirstlane(p.cu[seq]);
    const int L = __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);
    const uint32_t qrow = uint32_t(p.ld_qkv) * 2u, orow = uint32_t(p.ld_o) * 2u;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(p.dout + tok0 * p.ld_o + int64_t(head) * D, uint64_t(L) * orow);
    const __amdgpu_buffer_rsrc_t l_rs = make_rsrc(p.lse + int64_t(head) * p.T + tok0, uint64_t(L) * 4u);
    const __amdgpu_buffer_rsrc_t d_rs = make_rsrc(p.dsum + int64_t(head) * p.T + tok0, uint64_t(L) * 4u);

    // K and V rows of this wavefront's 32 keys: MFMA B operands of
    // S = Q K^T and dP = dO V^T (lane: key l32, dims 16kk + 8h .. +7).
    const int key0 = tile * kKvKeys + wave * 32;
    bf16x8_t kf[TL::KK], vf[TL::KK];
    {
        const uint32_t off = uint32_t(key0 + l32) * qrow + 16u * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk) {
            kf[kk] = __builtin_bit_cast(bf16x8_t, bload16(k_rs, off, 32u * kk));
            vf[kk] = __builtin_bit_cast(bf16x8_t, bload16(v_rs, off, 32u * kk));
        }
    }

    // Q/dO tiles are staged through registers (buffer loads of step t+1
    // issued before step t's products, written to the other LDS buffer after
    // them): unlike direct global->LDS loads, this leaves the transposed LDS
    // reads free of waits on the loads in flight.  Thread `tid` owns the
    // 16-byte chunks tid + 256j of each tile (row = chunk / KCH); threads 0..31
    // also carry 16 bytes of LSE or D.
    constexpr int kCh = kKvQ * TL::KCH / (64 * kKvWaves);    // chunks per thread per tile
    u32x4_t sq[kCh], so[kCh], sst;
    auto stage_load = [&](int t) {
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int ch = tid + 64 * kKvWaves * j;
            const uint32_t row = uint32_t(t * kKvQ + ch / TL::KCH), col = 16u * uint32_t(ch % TL::KCH);
            sq[j] = bload16(q_rs, row * qrow + col, 0);
            so[j] = bload16(do_rs, row * orow + col, 0);
        }
        if (tid < 32)
            sst = bload16(tid < 16 ? l_rs : d_rs, 16u * uint32_t(tid & 15), uint32_t(t) * kKvQ * 4u);
    };
    auto stage_store = [&](int stage) {
        unsigned char* base = smem + stage * TL::KV_STAGE;
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int ch = tid + 64 * kKvWaves * j;
            const int off = (ch / TL::KCH) * TL::X_ROW + 16 * (ch % TL::KCH);
            *reinterpret_cast<u32x4_t*>(base + off) = sq[j];
            *reinterpret_cast<u32x4_t*>(base + TL::QT_BYTES + off) = so[j];
        }
        if (tid < 32) *reinterpret_cast<u32x4_t*>(base + 2 * TL::QT_BYTES + 16 * tid) = sst;
    };

    f32x16_t dva[TL::EB], dka[TL::EB];
#pragma unroll
    for (int m = 0; m < TL::EB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dva[m][r] = dka[m][r] = 0.f;

    const int tr_rd = tr_offset<TL::X_ROW>(lane);
    const float c = p.c;
    const int nq = (L + kKvQ - 1) / kKvQ;
    stage_load(0);
    stage_store(0);
    __syncthreads();
    for (int t = 0; t < nq; ++t) {
        if (t + 1 < nq) stage_load(t + 1);
        const unsigned char* qt = smem + (t & 1) * TL::KV_STAGE;
        const unsigned char* ot = qt + TL::QT_BYTES;
        const float* st = reinterpret_cast<const float*>(qt + 2 * TL::QT_BYTES);

        // The step is one sequence of 64 MFMAs (32 for D = 64), with every LDS
        // operand read kPre MFMAs ahead and the VALU work of one block threaded
        // through the MFMAs of the other (a wavefront's VALU overlaps its own
        // MFMAs; there is no second wavefront on the SIMD to hide latency):
        //   ops [0, NA)      S, dP of block 0     (S = Q K^T, dP = dO V^T)
        //   ops [NA, 2NA)    S, dP of block 1     + P, dS of block 0
        //   ops [2NA, 2NA+NB)    dV, dK of block 0 + P, dS of block 1
        //   ops [2NA+NB, 2NA+2NB) dV, dK of block 1
        // After S and dP a lane holds one key (l32) and 16 queries of the block
        // (register r: query 8(r/4) + 4h + r%4); dV^T += dO^T P and dK^T += Q^T dS
        // take dO^T / Q^T from transposed LDS reads and P / dS as bf16 B operands.
        constexpr int NA = 2 * TL::KK;          // S and dP MFMAs of one 32-query block
        constexpr int NB = 4 * TL::EB;          // dV and dK MFMAs of one block
        constexpr int NOPS = 2 * NA + 2 * NB;
        constexpr int kPre = 6;
        constexpr int kUnits = 16;              // VALU units of one block (one register each)
        f32x16_t s[2], dp[2];
        bf16x8_t pk[2][2][2];                   // [block][16-query half][P, dS]
        f32x4_t l4[2][4], d4[2][4];
        // Every index below is a compile-time constant (integral_constant
        // arguments), so all register arrays stay in registers.
        auto frag = [&](auto opc) -> bf16x8_t {
            constexpr int op = decltype(opc)::value;
            if constexpr (op < 2 * NA) {        // 16-byte row reads of Q (S) or dO (dP)
                constexpr int b = op / NA, i = op % NA, kk = i >> 1;
                const unsigned char* tile = (i & 1) ? ot : qt;
                return *reinterpret_cast<const bf16x8_t*>(tile + (32 * b + l32) * TL::X_ROW + 32 * kk + 16 * hlf);
            } else {                            // transposed reads of dO^T (dV) or Q^T (dK)
                constexpr int b = (op - 2 * NA) / NB, j = (op - 2 * NA) % NB;
                constexpr int h2 = j / (2 * TL::EB), m = (j >> 1) % TL::EB;
                return tr_frag<TL::X_ROW>((j & 1) ? qt : ot, tr_rd, 2 * b + h2, m);
            }
        };
        auto mfma_op = [&](auto opc, const bf16x8_t& f) {
            constexpr int op = decltype(opc)::value;
            if constexpr (op < 2 * NA) {
                constexpr int b = op / NA, i = op % NA, kk = i >> 1;
                if constexpr (i & 1)
                    dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, vf[kk], kk == 0 ? f32x16_t{} : dp[b], 0, 0, 0);
                else
                    s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, kf[kk], kk == 0 ? f32x16_t{} : s[b], 0, 0, 0);
            } else {
                constexpr int b = (op - 2 * NA) / NB, j = (op - 2 * NA) % NB;
                constexpr int h2 = j / (2 * TL::EB), m = (j >> 1) % TL::EB;
                if constexpr (j & 1)
                    dka[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pk[b][h2][1], dka[m], 0, 0, 0);
                else
                    dva[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pk[b][h2][0], dva[m], 0, 0, 0);
            }
        };
        auto load_stats = [&](int b) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                l4[b][gq] = *reinterpret_cast<const f32x4_t*>(st + 32 * b + 8 * gq + 4 * hlf);
                d4[b][gq] = *reinterpret_cast<const f32x4_t*>(st + kKvQ + 32 * b + 8 * gq + 4 * hlf);
            }
        };
        // P = exp(tau S - LSE), dS = P (dP - D) for register u of block b;
        // after registers 7 and 15 the half's bf16 B operands are packed.
        auto v_unit = [&](auto bc, auto uc) {
            constexpr int b = decltype(bc)::value, u = decltype(uc)::value;
            constexpr int gq = u >> 2, i = u & 3;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][u], c, -l4[b][gq][i] * kLog2e));
            s[b][u] = pr;
            dp[b][u] = pr * (dp[b][u] - d4[b][gq][i]);
            if constexpr ((u & 7) == 7) {
                pk[b][u >> 3][0] = pack_chunk(s[b], u >> 3);
                pk[b][u >> 3][1] = pack_chunk(dp[b], u >> 3);
            }
        };
        load_stats(0);
        load_stats(1);
        bf16x8_t fr[kPre];
        [&]<int... P>(std::integer_sequence<int, P...>) {
            ((fr[P] = frag(std::integral_constant<int, P>{})), ...);
        }(std::make_integer_sequence<int, kPre>{});
        auto one_op = [&](auto opc) {
            constexpr int op = decltype(opc)::value;
            __builtin_amdgcn_sched_barrier(0);
            mfma_op(opc, fr[op % kPre]);
            if constexpr (op + kPre < NOPS) fr[op % kPre] = frag(std::integral_constant<int, op + kPre>{});
            // VALU of block 0 rides on the S/dP MFMAs of block 1, that of
            // block 1 on the dV/dK MFMAs of block 0
            if constexpr (op >= NA && op < 2 * NA) {
                constexpr int per = kUnits / NA;
                [&]<int... K>(std::integer_sequence<int, K...>) {
                    (v_unit(std::integral_constant<int, 0>{}, std::integral_constant<int, (op - NA) * per + K>{}), ...);
                }(std::make_integer_sequence<int, per>{});
            } else if constexpr (op >= 2 * NA && op < 2 * NA + NB) {
                constexpr int per = kUnits / NB;
                [&]<int... K>(std::integer_sequence<int, K...>) {
                    (v_unit(std::integral_constant<int, 1>{}, std::integral_constant<int, (op - 2 * NA) * per + K>{}), ...);
                }(std::make_integer_sequence<int, per>{});
            }
        };
        [&]<int... OPS>(std::integer_sequence<int, OPS...>) {
            (one_op(std::integral_constant<int, OPS>{}), ...);
        }(std::make_integer_sequence<int, NOPS>{});
        __builtin_amdgcn_sched_barrier(0);
        // the other buffer was last read in step t-1, which every wavefront
        // finished before the barrier that opened step t
        if (t + 1 < nq) stage_store((t + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane l32 owns key key0 + l32
    if (key0 + l32 < L) {
        const int64_t row = (tok0 + key0 + l32) * p.ld_d + int64_t(head) * D;
        store_rows_t<D>(p.dv + row, dva, 1.0f, hlf);
        store_rows_t<D>(p.dk + row, dka, p.scale, hlf);
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdParams p) {
    using TL = BT<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int seq, head, tile;
    if (!locate_unit(p.pre_q, p.n_seq, p.H, blockIdx.x, seq, head, tile)) return;
    seq = __builtin_amdgcn_readfirstlane(seq);
    head = __builtin_amdgcn_readfirstlane(head);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int64_t tok0 = __builtin_amdgcn_readfirstlane(p.cu[seq]);
    const int L = __builtin_amdgcn_readfirstlane(p.cu[seq + 1]) - int(tok0);
    const uint32_t qrow = uint32_t(p.ld_qkv) * 2u, orow = uint32_t(p.ld_o) * 2u;
    const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(p.q + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + tok0 * p.ld_qkv + int64_t(head) * D, uint64_t(L) * qrow);
    const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(p.dout + tok0 * p.ld_o + int64_t(head) * D, uint64_t(L) * orow);
    const __amdgpu_buffer_rsrc_t l_rs = make_rsrc(p.lse + int64_t(head) * p.T + tok0, uint64_t(L) * 4u);
    const __amdgpu_buffer_rsrc_t d_rs = make_rsrc(p.dsum + int64_t(head) * p.T + tok0, uint64_t(L) * 4u);

    // Q and dO rows of this wavefront's 32 queries: B operands of
    // S^T = K Q^T and dP^T = V dO^T; LSE and D of the lane's query.
    const int q0 = tile * kQRows + wave * 32;
    bf16x8_t qf[TL::KK], of[TL::KK];
    {
        const uint32_t qoff = uint32_t(q0 + l32) * qrow + 16u * hlf;
        const uint32_t ooff = uint32_t(q0 + l32) * orow + 16u * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk) {
            qf[kk] = __builtin_bit_cast(bf16x8_t, bload16(q_rs, qoff, 32u * kk));
            of[kk] = __builtin_bit_cast(bf16x8_t, bload16(do_rs, ooff, 32u * kk));
        }
    }
    const float nl = -__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(l_rs, uint32_t(q0 + l32) * 4u, 0, 0)) * kLog2e;
    const float dq_d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d_rs, uint32_t(q0 + l32) * 4u, 0, 0));

    // K/V tiles staged through registers one step ahead into two LDS
    // buffers (see the dK/dV kernel): thread `tid` owns chunks tid + 512j.
    constexpr int kCh = kQK * TL::KCH / (64 * kQWaves);
    u32x4_t sk[kCh], sv[kCh];
    auto stage_load = [&](int t) {
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int ch = tid + 64 * kQWaves * j;
            const uint32_t off = uint32_t(t * kQK + ch / TL::KCH) * qrow + 16u * uint32_t(ch % TL::KCH);
            sk[j] = bload16(k_rs, off, 0);
            sv[j] = bload16(v_rs, off, 0);
        }
    };
    auto stage_store = [&](int stage) {
        unsigned char* base = smem + stage * TL::Q_STAGE;
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
            const int ch = tid + 64 * kQWaves * j;
            *reinterpret_cast<u32x4_t*>(base + (ch / TL::KCH) * TL::X_ROW + 16 * (ch % TL::KCH)) = sk[j];
            *reinterpret_cast<u32x4_t*>(base + TL::KT_BYTES + (ch / TL::KCH) * TL::R_ROW + 16 * (ch % TL::KCH)) = sv[j];
        }
    };

    f32x16_t dqa[TL::EB];
#pragma unroll
    for (int m = 0; m < TL::EB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[m][r] = 0.f;

    const int tr_rd = tr_offset<TL::X_ROW>(lane);
    const float c = p.c;
    const int nk = (L + kQK - 1) / kQK;
    const int masked_tile = (L % kQK) != 0 ? nk - 1 : nk;
    stage_load(0);
    stage_store(0);
    __syncthreads();
    // Only the last key tile can need masking.  The steady steps are built
    // without the masking branch: a branch inside the sequence lets the
    // compiler gather the VALU work threaded before it into one block.
    auto step = [&](auto maskc, const int t) {
        constexpr bool kMask = decltype(maskc)::value;
        if (t + 1 < nk) stage_load(t + 1);
        const unsigned char* kt = smem + (t & 1) * TL::Q_STAGE;
        const unsigned char* vt = kt + TL::KT_BYTES;

        // One compile-time sequence per step (48 MFMAs for D = 128):
        //   ops [0, NA)           S^T, dP^T of key block 0
        //   ops [NA, 2NA)         S^T, dP^T of key block 1 + dS^T of block 0
        //   ops [2NA, 2NA+NB)     dQ^T += K^T dS^T for block 0 + dS^T of block 1
        //   ops [2NA+NB, 2NA+2NB) dQ^T for block 1
        // (lane: query l32; register r of a block: key 8(r/4) + 4h + r%4).
        constexpr int NA = 2 * TL::KK;
        constexpr int NB = 2 * TL::EB;
        constexpr int NOPS = 2 * NA + 2 * NB;
        constexpr int kPre = 4;
        constexpr int kUnits = 16;
        f32x16_t s[2], dp[2];
        bf16x8_t pk[2][2];                  // [key block][16-key half] dS^T as bf16 B operand
        auto frag = [&](auto opc) -> bf16x8_t {
            constexpr int op = decltype(opc)::value;
            if constexpr (op < 2 * NA) {    // 16-byte row reads of K (S^T) or V (dP^T)
                constexpr int b = op / NA, i = op % NA, kk = i >> 1;
                if constexpr (i & 1)
                    return *reinterpret_cast<const bf16x8_t*>(vt + (32 * b + l32) * TL::R_ROW + 32 * kk + 16 * hlf);
                else
                    return *reinterpret_cast<const bf16x8_t*>(kt + (32 * b + l32) * TL::X_ROW + 32 * kk + 16 * hlf);
            } else {                        // transposed reads of K^T
                constexpr int b = (op - 2 * NA) / NB, j = (op - 2 * NA) % NB;
                return tr_frag<TL::X_ROW>(kt, tr_rd, 2 * b + j / TL::EB, j % TL::EB);
            }
        };
        auto mfma_op = [&](auto opc, const bf16x8_t& f) {
            constexpr int op = decltype(opc)::value;
            if constexpr (op < 2 * NA) {
                constexpr int b = op / NA, i = op % NA, kk = i >> 1;
                if constexpr (i & 1)
                    dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, of[kk], kk == 0 ? f32x16_t{} : dp[b], 0, 0, 0);
                else
                    s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[kk], kk == 0 ? f32x16_t{} : s[b], 0, 0, 0);
            } else {
                constexpr int b = (op - 2 * NA) / NB, j = (op - 2 * NA) % NB;
                constexpr int m = j % TL::EB;
                dqa[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pk[b][j / TL::EB], dqa[m], 0, 0, 0);
            }
        };
        // keys past the end of the sequence (last tile only) get P = 0
        auto mask_block = [&](int b) {
            if constexpr (kMask) {
                if (t == masked_tile) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = t * kQK + 32 * b + 8 * (r >> 2) + 4 * hlf + (r & 3);
                        if (key >= L) s[b][r] = -INFINITY;
                    }
                }
            }
        };
        // dS^T = P^T (dP^T - D), P^T = exp(tau S^T - LSE), register u of block b
        auto v_unit = [&](auto bc, auto uc) {
            constexpr int b = decltype(bc)::value, u = decltype(uc)::value;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][u], c, nl));
            dp[b][u] = pr * (dp[b][u] - dq_d);
            if constexpr ((u & 7) == 7) pk[b][u >> 3] = pack_chunk(dp[b], u >> 3);
        };
        bf16x8_t fr[kPre];
        [&]<int... P>(std::integer_sequence<int, P...>) {
            ((fr[P] = frag(std::integral_constant<int, P>{})), ...);
        }(std::make_integer_sequence<int, kPre>{});
        auto one_op = [&](auto opc) {
            constexpr int op = decltype(opc)::value;
            if constexpr (op == NA) mask_block(0);
            if constexpr (op == 2 * NA) mask_block(1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_op(opc, fr[op % kPre]);
            if constexpr (op + kPre < NOPS) fr[op % kPre] = frag(std::integral_constant<int, op + kPre>{});
            if constexpr (op >= NA && op < 2 * NA) {
                constexpr int per = kUnits / NA;
                [&]<int... K>(std::integer_sequence<int, K...>) {
                    (v_unit(std::integral_constant<int, 0>{}, std::integral_constant<int, (op - NA) * per + K>{}), ...);
                }(std::make_integer_sequence<int, per>{});
            } else if constexpr (op >= 2 * NA && op < 2 * NA + NB) {
                constexpr int per = kUnits / NB;
                [&]<int... K>(std::integer_sequence<int, K...>) {
                    (v_unit(std::integral_constant<int, 1>{}, std::integral_constant<int, (op - 2 * NA) * per + K>{}), ...);
                }(std::make_integer_sequence<int, per>{});
            }
        };
        [&]<int... OPS>(std::integer_sequence<int, OPS...>) {
            (one_op(std::integral_constant<int, OPS>{}), ...);
        }(std::make_integer_sequence<int, NOPS>{});
        __builtin_amdgcn_sched_barrier(0);
        // the other buffer was last read in step t-1, finished by everyone
        // before the barrier that opened step t
        if (t + 1 < nk) stage_store((t + 1) & 1);
        __syncthreads();
    };
    for (int t = 0; t + 1 < nk; ++t) step(std::false_type{}, t);
    step(std::true_type{}, nk - 1);

    if (q0 + l32 < L) store_rows_t<D>(p.dq + (tok0 + q0 + l32) * p.ld_d + int64_t(head) * D, dqa, p.scale, hlf);
}

// One non-blocking side stream and a fork/join event pair per device,
// created on the first call that is not under stream capture (creating a
// stream is not allowed during capture); until then, and if creation fails,
// both kernels run on the caller's stream.  The mutex keeps one call's
// record/wait pairs together when several host threads launch at once (a
// wait binds to the event's latest record).
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
bool g_side_tried[kMaxDevices];
std::mutex g_side_mu;

// Caller holds g_side_mu.
SideStream* side_stream(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (!g_side_tried[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
        g_side_tried[dev] = true;
        SideStream s;
        if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&s.join, hipEventDisableTiming) == hipSuccess)
            g_side[dev] = s;
    }
    return g_side[dev].join ? &g_side[dev] : nullptr;
}

template <int D>
hipError_t launch_bwd_d(const AttnBwdArgs& a, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.dout = a.dout; p.lse = a.lse;
    p.dsum = reinterpret_cast<float*>(ws);
    p.pre_kv = reinterpret_cast<const int64_t*>(ws + ws_dsum_bytes(a.T, a.H));
    p.pre_q = reinterpret_cast<const int64_t*>(ws + ws_dsum_bytes(a.T, a.H) + ws_pre_bytes(a.n_seq));
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.cu = a.cu_seqlens;
    p.n_seq = a.n_seq; p.H = a.H; p.T = a.T;
    p.ld_qkv = a.ld_qkv; p.ld_o = a.ld_o; p.ld_d = a.ld_d;
    p.scale = a.softmax_scale;
    p.c = a.softmax_scale * kLog2e;

    hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seq,
                       const_cast<int64_t*>(p.pre_kv), const_cast<int64_t*>(p.pre_q));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int RPB = 256 / (D / 8);
    const int64_t rows = a.T * a.H;
    hipLaunchKernelGGL(bwd_dot_kernel<D>, dim3(unsigned((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                       a.o, a.dout, a.ld_o, p.dsum, a.T, a.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    static const hipError_t attr_kv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(BT<D>::KV_LDS));
    if (attr_kv != hipSuccess) return attr_kv;
    static const hipError_t attr_q = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(BT<D>::Q_LDS));
    if (attr_q != hipSuccess) return attr_q;
    // Upper bounds of the unit counts: sum_s ceil(L_s / n) <= T / n + n_seq.
    const int64_t units_kv = int64_t(a.H) * (a.T / kKvKeys + a.n_seq);
    const int64_t units_q = int64_t(a.H) * (a.T / kQRows + a.n_seq);
    // The dQ kernel runs beside the dK/dV kernel on a second stream: both
    // only read what the dot kernel wrote, and each alone leaves the last of
    // its ~3 rounds of work units on part of the chip.
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side = side_stream(stream);
    hipStream_t qs = side ? side->stream : stream;
    if (side) {
        if ((e = hipEventRecord(side->fork, stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(qs, side->fork, 0)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3(unsigned(units_q)), dim3(64 * kQWaves),
                       BT<D>::Q_LDS, qs, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3(unsigned(units_kv)), dim3(64 * kKvWaves),
                       BT<D>::KV_LDS, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (side) {
        if ((e = hipEventRecord(side->join, qs)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(stream, side->join, 0)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

size_t attn_bwd_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t /*D*/) {
    const int n = n_seq < 0 ? 0 : n_seq;
    return ws_dsum_bytes(T, H) + 2 * ws_pre_bytes(n);
}

hipError_t launch_varlen_attn_bwd(const AttnBwdArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_bwd_d<128>(a, stream);
    return launch_bwd_d<64>(a, stream);
}

}  // namespace mf
