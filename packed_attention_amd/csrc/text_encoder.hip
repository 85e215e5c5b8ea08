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
//  * attn_causal_kernel<D>: a unit of work is gb query heads of one
//    key/value group (gb = 4 when the group size allows it) times a slab of
//    128 / gb queries of one prompt, one wavefront per 32 queries of a head,
//    so the heads that share K and V share its tiles and, with gb = 4, all
//    four wavefronts stop at the same diagonal.  A one-workgroup prologue
//    writes one descriptor per (prompt, slab), sorted by key-tile count,
//    longest first.  Two persistent workgroups per CU walk that list in
//    snake order; each step is one key tile of 64, and the next step's tile
//    (this unit's next or the next unit's first) is fetched by direct
//    global->LDS loads into the other of two padded buffers while the
//    current one is used, so the pipeline does not drain between units.  The
//    next unit's Q is loaded into registers once the last tile's scores are
//    formed.  A unit's output waits in registers until the next unit's
//    first step, which stages it through the buffer that step is about to
//    fill and stores whole rows (one 16-byte chunk per lane, four rows per
//    instruction) before issuing its tile loads.  Per tile a wavefront computes S^T = K Q^T (each lane: one query,
//    16 keys per 32-key block), masks keys past the query or past the prompt
//    on the tiles that reach them, runs the online softmax with a lazily
//    raised reference max, and accumulates O^T += V^T P^T with V^T read
//    transposed from LDS (ds_read_b64_tr_b16) and P^T rounded to bf16 in
//    registers.
#include <algorithm>
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
constexpr int kCN = 64;                // keys per tile
constexpr int kSlabMin = 32;           // smallest query slab (four grouped heads)
// Workgroups per CU in the grid.  The LDS holds two, and the D = 128 kernel
// stays within 256 registers per lane (249 VGPRs), so both are resident, two
// wavefronts per SIMD; every register more than that would leave one.
constexpr int kWgPerCu = 2;
constexpr int kClasses = 1024;         // work classes (key-tile counts) of the longest-first order
static_assert(kClasses % 256 == 0, "whole classes per prologue thread");
constexpr float kRescale = 8.0f;       // lazy-rescale threshold (log2 units)
constexpr int kPrefetch = 4;           // MFMA operand fragments read ahead from LDS

template <int D>
struct CT {
    static constexpr int KK = D / 16;
    static constexpr int EB = D / 32;
    static constexpr int KCH = D / 8;                // 16-byte chunks per row
    static constexpr int K_UNITS = KCH + 1;          // K row: chunks + 1 pad (conflict-free row reads)
    static constexpr int V_UNITS = KCH + 4;          // V row: chunks + 4 pad (conflict-free transposed reads)
    static constexpr int K_ROW = 16 * K_UNITS;
    static constexpr int V_ROW = 16 * V_UNITS;
    static constexpr int K_BYTES = kCN * K_ROW;
    static constexpr int V_BYTES = kCN * V_ROW;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int LDS = 2 * STAGE;
    // direct loads per tile (64 lanes x 16 bytes each) and per wavefront
    static constexpr int K_DMA = kCN * K_UNITS / 64;
    static constexpr int V_DMA = kCN * V_UNITS / 64;
    static constexpr int K_DMA_W = (K_DMA + kCW - 1) / kCW;
    static constexpr int V_DMA_W = (V_DMA + kCW - 1) / kCW;
    static_assert(kCN * K_UNITS % 64 == 0 && kCN * V_UNITS % 64 == 0, "whole direct loads");
    static_assert(kWgPerCu * LDS <= 160 * 1024, "resident workgroups fit the LDS");
};

// Heads of one key/value group that share a workgroup: the largest of 4, 2, 1
// dividing the group size.  The workgroup's four wavefronts cover those heads
// times 128 / gb queries (a slab) of one prompt.
__host__ __device__ constexpr int heads_per_wg(int group) { return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1; }

// Key tiles that slab j (sq queries) of a prompt of length L walks.
__device__ __forceinline__ int slab_tiles(int L, int j, int sq) { return (min(L, j * sq + sq) - 1) / kCN + 1; }

// Slab descriptors {first token, prompt length, slab index, 0}, one per
// (prompt, slab), sorted by key-tile count, longest first (a counting sort;
// the order inside a class is arbitrary and does not affect any result);
// entry max_slabs holds the slab count.  One workgroup.
__global__ __launch_bounds__(256) void causal_slabs_kernel(const int32_t* __restrict__ cu, int n, int sq,
                                                           int max_slabs, int4* __restrict__ desc) {
    __shared__ int cls[kClasses];
    const int tid = threadIdx.x;
    for (int c = tid; c < kClasses; c += 256) cls[c] = 0;
    __syncthreads();
    const int per = (n + 255) / 256;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    for (int s = s0; s < s1; ++s) {
        const int L = cu[s + 1] - cu[s];
        for (int j = 0, ns = (L + sq - 1) / sq; j < ns; ++j) atomicAdd(&cls[min(slab_tiles(L, j, sq), kClasses - 1)], 1);
    }
    __syncthreads();
    // exclusive offsets of the classes, longest first: thread k owns classes
    // kClasses-1-4k .. kClasses-4-4k; a scan of the 256 partial sums
    constexpr int kPer = kClasses / 256;
    __shared__ int part[256];
    int own[kPer], sum = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        own[e] = cls[kClasses - 1 - (kPer * tid + e)];
        sum += own[e];
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 256; d *= 2) {
        const int v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int r = part[tid] - sum;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        cls[kClasses - 1 - (kPer * tid + e)] = r;
        r += own[e];
    }
    if (tid == 255) desc[max_slabs] = int4{r, 0, 0, 0};
    __syncthreads();
    for (int s = s0; s < s1; ++s) {
        const int a = cu[s], L = cu[s + 1] - a;
        for (int j = 0, ns = (L + sq - 1) / sq; j < ns; ++j)
            desc[atomicAdd(&cls[min(slab_tiles(L, j, sq), kClasses - 1)], 1)] = int4{a, L, j, 0};
    }
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
    const int4* desc;
    int max_slabs;
    int Hq, Hkv;
    int gb;             // heads per workgroup
    int hg;             // workgroups per slab: Hkv * (Hq / Hkv) / gb
    int64_t T, ld_q, ld_kv, ld_o;
    float c;            // softmax scale * log2(e)
};

// One unit of work as the workgroup sees it (all wavefront-uniform).
struct CUnit {
    int tok0, L, j, hgi;
};

template <int D>
__global__ __launch_bounds__(64 * kCW) void attn_causal_kernel(CausalParams p) {
    using TL = CT<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const int group = p.Hq / p.Hkv;
    const int ns = group / p.gb;                 // head groups per key/value head
    const int sq = 128 / p.gb;                   // queries per slab
    const int G = gridDim.x, b = blockIdx.x;
    const uint32_t qrow = uint32_t(p.ld_q) * 2u, kvrow = uint32_t(p.ld_kv) * 2u;
    const __amdgpu_buffer_rsrc_t desc_rs = make_rsrc(p.desc, uint64_t(p.max_slabs + 1) * 16u);
    const int W = __builtin_amdgcn_readfirstlane(int(bload16(desc_rs, 0, uint32_t(p.max_slabs) * 16u)[0])) * p.hg;

    // unit i of this workgroup: snake order over the longest-first list
    auto unit_of = [&](int i) { return i * G + ((i & 1) ? G - 1 - b : b); };
    // descriptor of unit i as a vector load (zeros, length 0, past the end)
    auto load_desc = [&](int i) -> u32x4_t {
        const int w = unit_of(i);
        u32x4_t d = bload16(desc_rs, 0, uint32_t(w < W ? w / p.hg : p.max_slabs + 1) * 16u);
        return d;
    };
    auto decode = [&](u32x4_t d, int i) {
        CUnit u;
        u.tok0 = __builtin_amdgcn_readfirstlane(int(d[0]));
        u.L = __builtin_amdgcn_readfirstlane(int(d[1]));
        u.j = __builtin_amdgcn_readfirstlane(int(d[2]));
        u.hgi = unit_of(i) % p.hg;
        if (unit_of(i) >= W) u.L = 0;
        return u;
    };
    auto kvh_of = [&](const CUnit& u) { return u.hgi / ns; };
    auto head_of = [&](const CUnit& u) { return kvh_of(u) * group + (u.hgi % ns) * p.gb + wave % p.gb; };
    auto q0_of = [&](const CUnit& u) { return u.j * sq + (wave / p.gb) * 32; };
    auto tiles_of = [&](const CUnit& u) { return (min(u.L, u.j * sq + sq) - 1) / kCN + 1; };

    // Q fragments of a unit: lane holds query q0 + l32 (B operand of S^T = K Q^T)
    auto q_load = [&](const CUnit& u, bf16x8_t* dst) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.q + int64_t(u.tok0) * p.ld_q + int64_t(head_of(u)) * D,
                                                    uint64_t(u.L) * qrow);
        const uint32_t off = uint32_t(q0_of(u) + l32) * qrow + 16u * hlf;
#pragma unroll
        for (int kk = 0; kk < TL::KK; ++kk) dst[kk] = __builtin_bit_cast(bf16x8_t, bload16(rs, off, 32u * kk));
    };

    // Direct global->LDS loads of a key tile.  Instruction n of a tile fills
    // LDS units [64n, 64n+64) of the padded K (or V) image: lane l fetches
    // unit 64n+l = (row, chunk); pad units fetch the row's last chunk again
    // (never read back).  Instruction n is issued by wavefront n % 4.  The
    // resource covers the prompt's rows of the key/value head and the tile
    // offset is the instruction's scalar offset, which the range check
    // includes, so rows past the prompt read as zeros.
    uint32_t k_off[TL::K_DMA_W], v_off[TL::V_DMA_W];
#pragma unroll
    for (int m = 0; m < TL::K_DMA_W; ++m) {
        const int u = 64 * (wave + kCW * m) + lane;
        k_off[m] = uint32_t(u / TL::K_UNITS) * kvrow + 16u * uint32_t(min(u % TL::K_UNITS, TL::KCH - 1));
    }
#pragma unroll
    for (int m = 0; m < TL::V_DMA_W; ++m) {
        const int u = 64 * (wave + kCW * m) + lane;
        v_off[m] = uint32_t(u / TL::V_UNITS) * kvrow + 16u * uint32_t(min(u % TL::V_UNITS, TL::KCH - 1));
    }
    auto stage = [&](const CUnit& u, int t, unsigned char* kb) {
        const int64_t base = int64_t(u.tok0) * p.ld_kv + int64_t(kvh_of(u)) * D;
        const uint64_t bytes = uint64_t(u.L) * kvrow;
        const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(p.k + base, bytes);
        const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(p.v + base, bytes);
        const uint32_t tile_off = uint32_t(t) * kCN * kvrow;   // range-checked like the lane offset
#pragma unroll
        for (int m = 0; m < TL::K_DMA_W; ++m)
            if (TL::K_DMA % kCW == 0 || wave + kCW * m < TL::K_DMA)
                dma16(k_rs, kb + 1024 * (wave + kCW * m), k_off[m], tile_off);
#pragma unroll
        for (int m = 0; m < TL::V_DMA_W; ++m)
            if (TL::V_DMA % kCW == 0 || wave + kCW * m < TL::V_DMA)
                dma16(v_rs, kb + TL::K_BYTES + 1024 * (wave + kCW * m), v_off[m], tile_off);
    };

    if (b >= W) return;
    CUnit cur = decode(load_desc(0), 0);
    bf16x8_t qf[TL::KK];
    q_load(cur, qf);
    stage(cur, 0, smem);
    CUnit nxt = decode(load_desc(1), 1);
    u32x4_t d2 = load_desc(2);
    __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): first tile, Q and descriptors in
    __syncthreads();

    const float c = p.c;
    const int k_rd = l32 * TL::K_ROW + hlf * 16;
    const int v_rd = (4 * hlf + ((lane & 15) >> 2)) * TL::V_ROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    f32x16_t oacc[TL::EB];          // set on each unit's first tile
    float m_run = -INFINITY, l_run = 0.f;
    int buf = 0;

    // A unit's output (bf16 rows and LSE) is held in registers and stored at
    // the start of the next unit's first step (or after the last step).  The
    // wavefront's 32 x D tile goes through its own slice of the LDS buffer
    // that the step's tile loads are about to fill (free since the previous
    // barrier; rows of 2D bytes, 16-byte chunk c of row r in slot
    // c ^ (r % (D/8))), and is read back along rows, so each store instruction
    // writes whole rows (64 lanes x 16 bytes) instead of 16 bytes of 32
    // rows.  A barrier then hands the buffer to the loads.
    static_assert(kCW * 32 * 2 * D <= TL::STAGE, "output tiles fit a stage");
    constexpr int kRowCh = D / 8;                   // 16-byte chunks per output row
    u32x4_t out_v[TL::EB][2];
    float out_lse = 0.f;
    int out_q0 = 0, out_L = 0, out_tok0 = 0, out_head = 0;
    bool out_pending = false;
    auto flush_out = [&](unsigned char* stg) {
        unsigned char* const wb = stg + wave * (32 * 2 * D);
#pragma unroll
        for (int m = 0; m < TL::EB; ++m)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                const int cidx = 4 * m + 2 * gp + hlf;
                *reinterpret_cast<u32x4_t*>(wb + l32 * (2 * D) + 16 * (cidx ^ (l32 & (kRowCh - 1)))) = out_v[m][gp];
            }
        constexpr int kRowsPer = 64 / kRowCh;       // rows one store instruction covers
#pragma unroll 1
        for (int k = 0; k < 32 / kRowsPer; ++k) {
            const int row = kRowsPer * k + lane / kRowCh, cidx = lane % kRowCh;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wb + row * (2 * D) + 16 * (cidx ^ (row & (kRowCh - 1))));
            if (out_q0 + row < out_L)
                st16(p.o + (int64_t(out_tok0) + out_q0 + row) * p.ld_o + int64_t(out_head) * D + 8 * cidx, v);
        }
        if (p.lse != nullptr && hlf == 0 && out_q0 + l32 < out_L)
            p.lse[int64_t(out_head) * p.T + out_tok0 + out_q0 + l32] = out_lse;
    };

    // One key tile t of the current unit on LDS buffer `buf`, with the next
    // tile (this unit's t+1 or, on the last tile, the next unit's first)
    // fetched into the other buffer.  First: the accumulators start at zero.
    // Last: the next unit's Q is loaded into qf once the scores are formed,
    // and the unit's output is written.
    // The buffer read (kt) and the one filled (nb) are restrict pointers: the
    // compiler then knows that the direct loads into nb do not feed this
    // step's LDS reads and does not wait for them before the first read.
    auto step = [&](auto first_c, auto last_c, const int t, const bool more, const unsigned char* __restrict__ kt,
                    unsigned char* __restrict__ nb) {
        constexpr bool kFirst = decltype(first_c)::value, kLast = decltype(last_c)::value;
        const unsigned char* const vt = kt + TL::K_BYTES;
        if constexpr (kFirst) {
            if (out_pending) {
                flush_out(nb);
                __syncthreads();
            }
        }
        // nb was last read in the previous step, finished by everyone before
        // the barrier that opened this one
        if (more) {
            if constexpr (kLast) stage(nxt, 0, nb);
            else stage(cur, t + 1, nb);
        }
        const int q0 = q0_of(cur);
        // S^T = K Q^T: two 32-key blocks (lane: query q0 + l32, register r:
        // key 32 b + 8 (r/4) + 4 h + r%4 of the tile)
        // fragment i: key block i % 2, 16-dim slice i / 2; kPrefetch of them
        // are read ahead of the MFMA that uses them
        auto kfrag = [&](int i) {
            return *reinterpret_cast<const bf16x8_t*>(kt + k_rd + (i & 1) * 32 * TL::K_ROW + (i >> 1) * 32);
        };
        f32x16_t sc[2];
        {
            bf16x8_t fr[kPrefetch];
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) fr[i] = kfrag(i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2 * TL::KK; ++i) {
                const bf16x8_t f = fr[i % kPrefetch];
                sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[i >> 1], i < 2 ? f32x16_t{} : sc[i & 1], 0, 0, 0);
                if (i + kPrefetch < 2 * TL::KK) fr[i % kPrefetch] = kfrag(i + kPrefetch);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (kLast) q_load(nxt, qf);     // length 0 past the end: zeros, no access
        // keys past the query (causal) or past the prompt: only on the tiles
        // that reach the wavefront's first query or the prompt's end
        if ((t + 1) * kCN - 1 > q0 || (t + 1) * kCN > cur.L) {
            const int lim = min(q0 + l32, cur.L - 1) - 4 * hlf - t * kCN;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * bb + 8 * (r >> 2) + (r & 3) > lim) sc[bb][r] = -INFINITY;
        }
        // online softmax, reference max raised lazily (numerator and
        // denominator share it, so the result is the same softmax); on a
        // unit's first tile the max is taken as it is
        float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = (bb == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, sc[bb][r]);
        mx = half_max32(mx) * c;
        if constexpr (kFirst) {
            m_run = mx;
        } else {
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
        }
        float lsum = 0.f;
        bf16x8_t pf[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int bb = cc >> 1, r0 = 8 * (cc & 1);
            float e[8];
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                e[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[bb][r0 + ii], c, -m_run));
                lsum += e[ii];
            }
            u32x4_t u;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) u[ii] = pack_bf16x2(e[2 * ii], e[2 * ii + 1]);
            pf[cc] = __builtin_bit_cast(bf16x8_t, u);
        }
        l_run = kFirst ? lsum : l_run + lsum;
        // O^T += V^T P^T over the four 16-key chunks (fragment jj: chunk
        // jj / EB, 32-dim block jj % EB), kPrefetch fragments read ahead
        auto vfrag = [&](int jj) {
            const unsigned char* ad = vt + v_rd + (jj / TL::EB) * 16 * TL::V_ROW + (jj % TL::EB) * 64;
            const s16x4_t lo = lds_read_tr16_b64(ad);
            const s16x4_t hi = lds_read_tr16_b64(ad + 8 * TL::V_ROW);
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        {
            bf16x8_t fr[kPrefetch];
#pragma unroll
            for (int jj = 0; jj < kPrefetch; ++jj) fr[jj] = vfrag(jj);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < 4 * TL::EB; ++jj) {
                oacc[jj % TL::EB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    fr[jj % kPrefetch], pf[jj / TL::EB], (kFirst && jj < TL::EB) ? f32x16_t{} : oacc[jj % TL::EB], 0, 0, 0);
                if (jj + kPrefetch < 4 * TL::EB) fr[jj % kPrefetch] = vfrag(jj + kPrefetch);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (kLast) {
            // the unit's output rows (queries inside the prompt) and LSE,
            // stored by the next unit's first step (or after the loop)
            const float l_tot = half_sum32(l_run);
            const float inv = 1.0f / l_tot;
            // lane (q, h) holds dims 8g + 4h + 0..3 of block m; swapping the
            // g = 2gp + 1 values of lanes q with the g = 2gp values of lanes
            // q + 32 (v_permlane32_swap) leaves lane (q, h) with dims
            // 16gp + 8h + 0..7, so each store writes 32 contiguous bytes per row
#pragma unroll
            for (int m = 0; m < TL::EB; ++m)
#pragma unroll
                for (int gp = 0; gp < 2; ++gp) {
                    uint32_t x[2], y[2];
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        x[w] = pack_bf16x2(oacc[m][8 * gp + 2 * w] * inv, oacc[m][8 * gp + 2 * w + 1] * inv);
                        y[w] = pack_bf16x2(oacc[m][8 * gp + 4 + 2 * w] * inv, oacc[m][8 * gp + 4 + 2 * w + 1] * inv);
                        const auto r = __builtin_amdgcn_permlane32_swap(x[w], y[w], false, false);
                        x[w] = r[0];
                        y[w] = r[1];
                    }
                    out_v[m][gp] = u32x4_t{x[0], x[1], y[0], y[1]};
                }
            out_lse = m_run * 0.69314718055994531f + logf(l_tot);
            out_q0 = q0;
            out_L = cur.L;
            out_tok0 = cur.tok0;
            out_head = head_of(cur);
            out_pending = true;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): the next tile (and Q) landed
        __syncthreads();
    };
    auto run = [&](auto first_c, auto last_c, const int t, const bool more) {
        step(first_c, last_c, t, more, smem + buf * TL::STAGE, smem + (buf ^ 1) * TL::STAGE);
        buf ^= 1;
    };

    for (int i = 0;;) {
        const int nt = tiles_of(cur);
        const bool more = nxt.L > 0;
        if (nt == 1) {
            run(std::true_type{}, std::true_type{}, 0, more);
        } else {
            run(std::true_type{}, std::false_type{}, 0, true);
            for (int t = 1; t + 1 < nt; ++t) run(std::false_type{}, std::false_type{}, t, true);
            run(std::false_type{}, std::true_type{}, nt - 1, more);
        }
        if (!more) {
            flush_out(smem);        // both buffers are free after the last barrier
            break;
        }
        // next unit: its first tile is in LDS and its Q in registers; fetch
        // the descriptor of the one after the next
        ++i;
        cur = nxt;
        nxt = decode(d2, i + 1);
        d2 = load_desc(i + 2);
    }
}

template <int D>
hipError_t launch_causal_d(const CausalAttnArgs& a, hipStream_t stream) {
    CausalParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.lse = a.lse;
    p.desc = static_cast<const int4*>(a.workspace);
    p.Hq = a.Hq; p.Hkv = a.Hkv;
    p.gb = heads_per_wg(a.Hq / a.Hkv);
    p.hg = a.Hkv * (a.Hq / a.Hkv / p.gb);
    p.T = a.T; p.ld_q = a.ld_q; p.ld_kv = a.ld_kv; p.ld_o = a.ld_o;
    p.c = a.softmax_scale * 1.4426950408889634f;
    const int sq = 128 / p.gb;
    // upper bound of the slab count: sum_s ceil(L_s / sq) <= T / sq + n_seq
    const int64_t max_slabs = a.T / sq + a.n_seq;
    if (max_slabs * p.hg > INT32_MAX / 2) return hipErrorInvalidValue;
    p.max_slabs = int(max_slabs);
    const int cus = device_cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL(causal_slabs_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seq, sq,
                       int(max_slabs), static_cast<int4*>(a.workspace));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_causal_kernel<D>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, CT<D>::LDS);
    if (attr != hipSuccess) return attr;
    const int64_t grid = std::min<int64_t>(int64_t(kWgPerCu) * cus, max_slabs * p.hg);
    hipLaunchKernelGGL(attn_causal_kernel<D>, dim3(unsigned(grid)), dim3(64 * kCW), CT<D>::LDS, stream, p);
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

size_t causal_attn_workspace_bytes(int32_t n_seq, int64_t T) {
    if (n_seq < 0 || T < 0) return 0;
    // one descriptor per slab of the smallest size, then the slab count
    return size_t(T / kSlabMin + n_seq + 1) * sizeof(int4);
}

hipError_t launch_varlen_attn_causal(const CausalAttnArgs& a, hipStream_t stream) {
    if (a.T == 0 || a.n_seq == 0) return hipSuccess;
    return a.D == 128 ? launch_causal_d<128>(a, stream) : launch_causal_d<64>(a, stream);
}

}  // namespace mf
