// Backward of the fused elementwise kernels (gfx950): adaLN modulation +
// multi-axis RoPE of q and k, and the gated residual with the fused next
// adaLN.  The pages train the model with these fused kernels (picx.dev
// summary of Mage-Flow, Methodology > Training Infrastructure; gist.science
// "Resumo Tecnico: Mage-Flow", Metodologia > 3. Otimizacao de Nivel de
// Sistema > Kernels Fundidos); the gradients are the chain rule of the
// forward steps:
//   RoPE:      each pair's gradient turns back by -phi;
//   modulate:  u = xh (1 + scale) + shift, xh = (x - mu) / sigma:
//              gx = du (1 + scale), dx = (gx - mean gx - xh mean(gx xh)) / sigma,
//              dshift[r] += du, dscale[r] += du xh;
//   residual:  y = x + gate o, z = LN(y)(1 + scale2) + shift2:
//              dyt = dy + LN-backward(dz (1 + scale2)), dx = dyt,
//              do = gate dyt, dgate[r] += dyt o, dshift2[r] += dz,
//              dscale2[r] += dz yh.
//
// Layout and mapping.  Each call runs two kernels and a reduction:
//  * the per-token outputs (dq, dk; dx, do) with the forward kernels'
//    mappings (modulate + RoPE: one wavefront per q or k row, statistics
//    inside the wavefront; gated residual: one workgroup per token, one
//    16-byte chunk per thread, LayerNorm reductions through LDS), which also
//    write each row's fp32 statistics (4 floats per token);
//  * the per-row sums over tokens (dshift, dscale; dgate, dshift2,
//    dscale2): one lane per 8-channel chunk walks a run of kSumRun tokens,
//    reads the rows again and recomputes the fp32 gradients from them and
//    the statistics, so the sums see the same fp32 values as the outputs.
//    A run's tokens in order split into segments of equal adaLN row; each
//    segment's sums are one entry (row tag + NA x C fp32) at the run's next
//    entry position (run r owns positions r R .. r R + R - 1);
//  * a segmented reduction over the entries in token order: each level
//    adds the entries of kFanIn consecutive groups of the level below,
//    merging neighbours of equal row, and writes the merged entries
//    compactly at the start of its own range; the last level (at most
//    kRootFan groups below it) adds its entries to the zeroed output rows.
//    One thread per channel and each level a launch of its own, so every
//    row sum is added in one fixed order: the row sums are bitwise
//    reproducible, as every per-token output is.  A row whose tokens are not
//    contiguous gets one entry per stretch, added in token order.
// Modulate + RoPE rows of more than 3072 channels keep a single kernel: a
// workgroup walks a run of kRun tokens one row at a time (thread per chunk,
// statistics by workgroup reductions) and writes its segment entries the
// same way.
#include <cmath>

#include "mf_device.h"
#include "mf_internal.h"

namespace mf {
namespace {

constexpr int kRun = 4;          // tokens per workgroup (wide rows)
constexpr int kFanIn = 16;       // groups merged per reduction level
constexpr int kRootFan = 128;    // at most this many groups below the last level
constexpr int kMaxLevels = 6;     // 128 x 16^5 runs
constexpr int kRedThreads = 256; // channels per reduction workgroup

// Zeros n floats at each of up to three arrays (blockIdx.y picks the array;
// nullptr entries are skipped), one launch for all of a call's row sums.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p0, float* __restrict__ p1,
                                                        float* __restrict__ p2, int64_t n) {
    float* const p = blockIdx.y == 0 ? p0 : blockIdx.y == 1 ? p1 : p2;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (p != nullptr && i < n) p[i] = 0.f;
}

hipError_t zero_f32(float* p0, float* p1, float* p2, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256), 3), dim3(256), 0, stream, p0, p1, p2, n);
    return hipGetLastError();
}

// Workgroup sum of N values per thread; every thread receives the totals.
// `red` holds 2 * N * 16 floats; successive calls must alternate `buf`
// (0, 1, 0, ...) so that one barrier per call suffices.
template <int N>
__device__ __forceinline__ void wg_sum(float (&v)[N], float* red, int buf) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = (blockDim.x + 63) >> 6;
    float* r = red + buf * N * 16;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float s = wave_sum(v[k]);
        if (lane == 0) r[k * 16 + wave] = s;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += r[k * 16 + w];
        v[k] = s;
    }
}

// ---------------------------------------------------------------------------
// Row sums: segment entries and their reduction
// ---------------------------------------------------------------------------
// Workspace of one call, each part 256-byte aligned:
//   tag0 int32 [P], cnt0 int32 [n_runs]: the runs' entries (P = n_runs R);
//   tags int32 [2][n_cb][P]: entry rows of the levels (odd / even levels);
//   cnts int32 [n_cb][n_cnt]: entries per group of each level;
//   vals fp32 [P][NA][C]: the entries' sums, reduced in place level by level;
//   stats fp32 [T][4]: the per-token statistics of the two-kernel forms.
struct SegLayout {
    int64_t n_runs = 0, P = 0, n_cnt = 0;
    int R = 0, NA = 0, C = 0, n_cb = 0, n_levels = 0;
    int64_t groups[kMaxLevels + 1] = {};   // groups of level k (k = 0: the runs)
    int64_t span[kMaxLevels + 1] = {};     // runs per group of level k
    int64_t cnt_off[kMaxLevels + 1] = {};  // level k's counts in cnts
    size_t off_tag0 = 0, off_cnt0 = 0, off_tags = 0, off_cnts = 0, off_vals = 0, off_stats = 0, total = 0;
};

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

SegLayout seg_layout(int64_t T, int C, int NA, int R) {
    SegLayout L;
    L.R = R;
    L.NA = NA;
    L.C = C;
    L.n_runs = (T + R - 1) / R;
    L.P = L.n_runs * R;
    L.n_cb = (C + kRedThreads - 1) / kRedThreads;
    L.groups[0] = L.n_runs;
    L.span[0] = 1;
    int k = 0;
    // levels of kFanIn until at most kRootFan groups remain, then the root
    while (L.groups[k] > kRootFan && k + 1 < kMaxLevels) {
        ++k;
        L.groups[k] = (L.groups[k - 1] + kFanIn - 1) / kFanIn;
        L.span[k] = L.span[k - 1] * kFanIn;
        L.cnt_off[k] = L.n_cnt;
        L.n_cnt += L.groups[k];
    }
    ++k;
    L.groups[k] = L.n_runs > 0 ? 1 : 0;
    L.span[k] = L.n_runs;
    L.n_levels = k;
    size_t b = 0;
    L.off_tag0 = b;  b += align256(size_t(L.P) * 4);
    L.off_cnt0 = b;  b += align256(size_t(L.n_runs) * 4);
    L.off_tags = b;  b += align256(size_t(2) * L.n_cb * L.P * 4);
    L.off_cnts = b;  b += align256(size_t(L.n_cb) * size_t(L.n_cnt > 0 ? L.n_cnt : 1) * 4);
    L.off_vals = b;  b += align256(size_t(L.P) * NA * C * 4);
    L.off_stats = b; b += align256(size_t(T) * 16);
    L.total = b;
    return L;
}

struct SegArgs {
    const int32_t* tag0;
    const int32_t* cnt0;
    int32_t* tags;
    int32_t* cnts;
    float* vals;
    float* out[3];
    int64_t P;
    int n_cnt, R, C, n_cb, n_levels, n_rows;
    int32_t groups[kMaxLevels + 1];
    int32_t span[kMaxLevels + 1];
    int32_t cnt_off[kMaxLevels + 1];
};

SegArgs seg_args(const SegLayout& L, void* ws, int n_rows, float* o0, float* o1, float* o2) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    SegArgs a = {};
    a.tag0 = reinterpret_cast<const int32_t*>(w + L.off_tag0);
    a.cnt0 = reinterpret_cast<const int32_t*>(w + L.off_cnt0);
    a.tags = reinterpret_cast<int32_t*>(w + L.off_tags);
    a.cnts = reinterpret_cast<int32_t*>(w + L.off_cnts);
    a.vals = reinterpret_cast<float*>(w + L.off_vals);
    a.out[0] = o0;
    a.out[1] = o1;
    a.out[2] = o2;
    a.P = L.P;
    a.R = L.R;
    a.C = L.C;
    a.n_cb = L.n_cb;
    a.n_levels = L.n_levels;
    a.n_rows = n_rows;
    a.n_cnt = int(L.n_cnt);
    for (int k = 0; k <= kMaxLevels; ++k) {
        a.groups[k] = int32_t(L.groups[k]);
        a.span[k] = int32_t(L.span[k]);
        a.cnt_off[k] = int32_t(L.cnt_off[k]);
    }
    return a;
}

// Level k of the reduction, one launch per level: workgroup (g, cb) merges,
// in order, the entries of the groups of level k - 1 below group g (level 0:
// the runs), channels [256 cb, 256 cb + 256).  Neighbouring entries of equal
// row are added; the merged entries go compactly to the start of group g's
// range (in place: each thread reads and writes only its own channel, and an
// entry is written only after every entry before it has been read), or, at
// the last level, are added to the output rows (zeroed by the kernel that
// wrote the runs' entries), which only this thread writes for its channel.
// A child's first entry sits at the start of its range whatever its count,
// so the children are taken kB at a time: one round of loads brings child
// j's count and first row to lane j of every wavefront (read back as scalars
// with readlane) and every thread's values of the children's first entries;
// further entries of a child (a row change inside it) are loaded one by one.
template <int NA>
constexpr int batch_children() { return NA >= 3 ? 16 : NA == 2 ? 32 : 64; }

template <int NA>
__global__ __launch_bounds__(kRedThreads) void seg_level_kernel(SegArgs a, int k) {
    constexpr int kB = batch_children<NA>();   // children per round of loads
    static_assert(kB <= kWave, "one child per lane");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cb = blockIdx.y;
    const int c = cb * kRedThreads + tid;
    const bool live = c < a.C;
    const int cc = live ? c : a.C - 1;     // the channel the loads use
    const int64_t g = blockIdx.x;
    const bool top = k == a.n_levels;
    const int fan = top ? int(a.groups[k - 1]) : kFanIn;
    const int64_t ch0 = g * fan;
    const int n_ch = int((ch0 + fan < a.groups[k - 1] ? ch0 + fan : a.groups[k - 1]) - ch0);
    const int64_t child_span = int64_t(a.span[k - 1]) * a.R;   // positions per child
    const int64_t out_base = g * int64_t(a.span[k]) * a.R;
    const int32_t* in_tags = k == 1 ? a.tag0 : a.tags + ((k - 1) & 1) * int64_t(a.n_cb) * a.P + cb * a.P;
    int32_t* out_tags = a.tags + (k & 1) * int64_t(a.n_cb) * a.P + cb * a.P;
    const int32_t* in_cnt = k == 1 ? a.cnt0 : a.cnts + int64_t(cb) * a.n_cnt + a.cnt_off[k - 1];
    float acc[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) acc[x] = 0.f;
    int cur = -1;
    int nout = 0;
    auto emit = [&]() {
        if (top) {
            if (live)
#pragma unroll
                for (int x = 0; x < NA; ++x) a.out[x][int64_t(cur) * a.C + c] += acc[x];
        } else {
            const int64_t pos = out_base + nout;
            if (live)
#pragma unroll
                for (int x = 0; x < NA; ++x) a.vals[(pos * NA + x) * a.C + c] = acc[x];
            if (tid == 0) out_tags[pos] = cur;
        }
        ++nout;
    };
    auto merge = [&](int tag, const float (&v)[NA]) {
        if (tag != cur) {
            if (cur >= 0) emit();
            cur = tag;
#pragma unroll
            for (int x = 0; x < NA; ++x) acc[x] = 0.f;
        }
#pragma unroll
        for (int x = 0; x < NA; ++x) acc[x] += v[x];
    };
    for (int b0 = 0; b0 < n_ch; b0 += kB) {
        const int nb = n_ch - b0 < kB ? n_ch - b0 : kB;
        int my_cnt = 0, my_tag = -1;
        if (lane < nb) {
            const int64_t ch = ch0 + b0 + lane;
            my_cnt = in_cnt[ch];
            my_tag = in_tags[ch * child_span];
        }
        // unconditional loads (a clamped child and channel past the ends;
        // those values go unused), so the batch is one round of loads
        float v[kB][NA];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t ch = ch0 + b0 + (j < nb ? j : nb - 1);
#pragma unroll
            for (int x = 0; x < NA; ++x) v[j][x] = a.vals[(ch * child_span * NA + x) * a.C + cc];
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int n = __builtin_amdgcn_readlane(my_cnt, j);   // 0 past the batch
            if (n > 0) merge(__builtin_amdgcn_readlane(my_tag, j), v[j]);
            for (int i = 1; i < n; ++i) {
                const int64_t pos = (ch0 + b0 + j) * child_span + i;
                float w[NA];
#pragma unroll
                for (int x = 0; x < NA; ++x) w[x] = a.vals[(pos * NA + x) * a.C + cc];
                merge(in_tags[pos], w);
            }
        }
    }
    if (cur >= 0) emit();
    if (!top && tid == 0) a.cnts[int64_t(cb) * a.n_cnt + a.cnt_off[k] + g] = nout;
}

template <int NA>
hipError_t reduce_segments(const SegLayout& L, void* ws, int n_rows, float* o0, float* o1, float* o2,
                           hipStream_t stream) {
    // the last level stages at most kRootFan children (reached for any T
    // below 128 x 16^5 runs)
    if (L.groups[L.n_levels - 1] > kRootFan) return hipErrorInvalidValue;
    const SegArgs args = seg_args(L, ws, n_rows, o0, o1, o2);
    for (int k = 1; k <= L.n_levels; ++k) {
        hipLaunchKernelGGL(seg_level_kernel<NA>, dim3(unsigned(L.groups[k]), unsigned(L.n_cb)), dim3(kRedThreads), 0,
                           stream, args, k);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Where a run writes its entries: run r's entry i at position r R + i.
// The same kernel zeroes the output rows (the reduction's last level adds
// into them), spread over all its threads.
struct SegLeaf {
    int32_t* tag0;
    int32_t* cnt0;
    float* vals;
    float* out[3];
    int64_t n_out;      // floats per output array (n_rows x C)
};

SegLeaf seg_leaf(const SegLayout& L, void* ws, int n_rows, float* o0, float* o1, float* o2) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    return SegLeaf{reinterpret_cast<int32_t*>(w + L.off_tag0), reinterpret_cast<int32_t*>(w + L.off_cnt0),
                   reinterpret_cast<float*>(w + L.off_vals), {o0, o1, o2}, int64_t(n_rows) * L.C};
}

__device__ __forceinline__ void zero_outputs(const SegLeaf& leaf) {
    const int64_t nthreads = int64_t(gridDim.x) * gridDim.y * blockDim.x;
    const int64_t i0 = (int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (int x = 0; x < 3; ++x)
        if (leaf.out[x] != nullptr)
            for (int64_t i = i0; i < leaf.n_out; i += nthreads) leaf.out[x][i] = 0.f;
}

// One segment's sums (8 channels of NA arrays) to the run's next entry.
template <int NA>
__device__ __forceinline__ void put_entry(float (&p)[NA][8], float* vals, int64_t pos, int C, int c0, bool live) {
    if (live)
#pragma unroll
        for (int x = 0; x < NA; ++x) {
            float* v = vals + (pos * NA + x) * C + c0;
            *reinterpret_cast<f32x4_t*>(v) = f32x4_t{p[x][0], p[x][1], p[x][2], p[x][3]};
            *reinterpret_cast<f32x4_t*>(v + 4) = f32x4_t{p[x][4], p[x][5], p[x][6], p[x][7]};
        }
#pragma unroll
    for (int x = 0; x < NA; ++x)
#pragma unroll
        for (int j = 0; j < 8; ++j) p[x][j] = 0.f;
}

// The two-kernel forms' sums workgroups take kRunsPerBlock runs of kSumRun
// tokens, one wavefront each, and merge them before they finish: each
// wavefront writes its run's entries (positions of its run) and their rows
// to LDS, then one thread per channel adds the workgroup's entries in token
// order and writes the merged entries compactly at the workgroup's range
// (kLeafSpan positions), so the reduction starts from one group per
// kLeafSpan tokens.  The first entry of every run is loaded in one round;
// further entries of a run (a row change inside it) one by one.  Lane w
// holds run w's count and first row, read back as scalars.
constexpr int kSumRun = 8;                            // tokens per sums wavefront
constexpr int kRunsPerBlock = 16;                     // wavefronts per sums workgroup
constexpr int kLeafSpan = kSumRun * kRunsPerBlock;    // positions (tokens) per sums workgroup
constexpr int kSumChannels = kWave * 8;               // channels per sums workgroup

template <int NA>
__device__ __forceinline__ void merge_block_runs(const SegLeaf& leaf, const int* s_cnt,
                                                 const int (*s_tag)[kSumRun], int C) {
    const int t = threadIdx.x;
    const int ch = blockIdx.y * kSumChannels + t;
    const bool live = t < kSumChannels && ch < C;
    const int cc = live ? ch : C - 1;      // the channel the loads use
    const int64_t base = int64_t(blockIdx.x) * kLeafSpan;
    // unconditional loads of every run's first entry (values of runs without
    // entries go unused), so they are one round of loads
    float v[kRunsPerBlock][NA];
#pragma unroll
    for (int w = 0; w < kRunsPerBlock; ++w)
#pragma unroll
        for (int x = 0; x < NA; ++x) v[w][x] = leaf.vals[((base + w * kSumRun) * NA + x) * C + cc];
    float acc[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) acc[x] = 0.f;
    int cur = -1;
    int nout = 0;
    auto emit = [&]() {
        const int64_t pos = base + nout;
        if (live)
#pragma unroll
            for (int x = 0; x < NA; ++x) leaf.vals[(pos * NA + x) * C + ch] = acc[x];
        if (blockIdx.y == 0 && t == 0) leaf.tag0[pos] = cur;
        ++nout;
    };
    auto merge = [&](int tag, const float (&w)[NA]) {
        if (tag != cur) {
            if (cur >= 0) emit();
            cur = tag;
#pragma unroll
            for (int x = 0; x < NA; ++x) acc[x] = 0.f;
        }
#pragma unroll
        for (int x = 0; x < NA; ++x) acc[x] += w[x];
    };
    // run w's count and first row in lane w, read back as scalars
    const int lane = t & 63;
    const int my_cnt = lane < kRunsPerBlock ? s_cnt[lane] : 0;
    const int my_tag = lane < kRunsPerBlock ? s_tag[lane][0] : -1;
#pragma unroll
    for (int w = 0; w < kRunsPerBlock; ++w) {
        const int n = __builtin_amdgcn_readlane(my_cnt, w);
        if (n > 0) merge(__builtin_amdgcn_readlane(my_tag, w), v[w]);
        for (int i = 1; i < n; ++i) {
            const int64_t pos = base + w * kSumRun + i;
            float u[NA];
#pragma unroll
            for (int x = 0; x < NA; ++x) u[x] = leaf.vals[(pos * NA + x) * C + cc];
            merge(s_tag[w][i], u);
        }
    }
    if (cur >= 0) emit();
    if (blockIdx.y == 0 && t == 0) leaf.cnt0[blockIdx.x] = nout;
}

// ---------------------------------------------------------------------------
// modulate + RoPE backward
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void modulate_rope_bwd_kernel(ModRopeBwdArgs a, SegLeaf leaf) {
    __shared__ float red[2 * 4 * 16];
    if (a.scale != nullptr) zero_outputs(leaf);   // RoPE only: no row sums
    const int C = a.H * a.D;
    const int ci = threadIdx.x;                 // this thread's chunk
    const bool live = ci < (C >> 3);
    const int c0 = 8 * ci;
    const bool mod = a.scale != nullptr;
    const float invC = 1.0f / float(C);
    const int e0 = c0 % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    double th[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) th[j] = a.theta_turns[e0 / 2 + j];
    const int64_t t_begin = int64_t(blockIdx.x) * kRun;
    const int64_t t_end = t_begin + kRun < a.T ? t_begin + kRun : a.T;
    float part[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[0][j] = part[1][j] = 0.f;
    int cur = -1;
    int n_ent = 0;
    // the finished segment of row `row` becomes the run's next entry (a row
    // outside the table adds nothing)
    auto flush = [&](int row) {
        if (row >= 0 && row < a.n_rows) {
            const int64_t pos = int64_t(blockIdx.x) * kRun + n_ent;
            put_entry<2>(part, leaf.vals, pos, C, c0, live);
            if (threadIdx.x == 0) leaf.tag0[pos] = row;
            ++n_ent;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) part[0][j] = part[1][j] = 0.f;
        }
    };
    int buf = 0;

    // rows of token t: output gradients of q and k, then q and k
    auto load = [&](int64_t t, u32x4_t (&r)[4]) {
        if (live) {
            r[0] = ld16(a.dq_out + t * a.ld_gout + c0);
            r[1] = ld16(a.dk_out + t * a.ld_gout + c0);
            if (mod) {
                r[2] = ld16(a.q_in + t * a.ld_in + c0);
                r[3] = ld16(a.k_in + t * a.ld_in + c0);
            }
        }
    };
    u32x4_t nxt[4] = {};
    load(t_begin, nxt);
    for (int64_t t = t_begin; t < t_end; ++t) {
        u32x4_t row[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) row[i] = nxt[i];
        if (t + 1 < t_end) load(t + 1, nxt);

        // gradient with respect to the RoPE input: each pair turned back
        float g[2][8];
        {
            const double p = double(a.pos[3 * t + axis]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double turns = p * th[j];
                const float f = float(turns - rint(turns));
                const float s = __builtin_amdgcn_sinf(f), c = __builtin_amdgcn_cosf(f);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const float h0 = bf_lo(row[x][j]), h1 = bf_hi(row[x][j]);
                    g[x][2 * j] = h0 * c + h1 * s;
                    g[x][2 * j + 1] = -h0 * s + h1 * c;
                }
            }
        }
        uint16_t* const dst[2] = {a.dq_in + t * a.ld_gin + c0, a.dk_in + t * a.ld_gin + c0};
        if (!mod) {
            if (live) {
                st16(dst[0], pack8(g[0]));
                st16(dst[1], pack8(g[1]));
            }
            continue;
        }
        const int m = a.mod_row[t];
        const bool mok = m >= 0 && m < a.n_rows;      // a row outside the table reads zeros, adds nothing
        if (m != cur) {
            flush(cur);
            cur = m;
        }
        float x[2][8];
        unpack8(row[2], x[0]);
        unpack8(row[3], x[1]);
        // LayerNorm statistics of the q and k rows (fp32, two passes)
        float st[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            st[0] += x[0][j];
            st[1] += x[1][j];
        }
        wg_sum<4>(st, red, buf);
        buf ^= 1;
        const float mu[2] = {st[0] * invC, st[1] * invC};
        float vr[4] = {0.f, 0.f, 0.f, 0.f};
        if (live)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                vr[0] += (x[0][j] - mu[0]) * (x[0][j] - mu[0]);
                vr[1] += (x[1][j] - mu[1]) * (x[1][j] - mu[1]);
            }
        wg_sum<4>(vr, red, buf);
        buf ^= 1;
        const float rs[2] = {rsqrtf(vr[0] * invC + a.eps), rsqrtf(vr[1] * invC + a.eps)};
        float sc[8];
        unpack8(live && mok ? ld16(a.scale + int64_t(m) * C + c0) : u32x4_t{}, sc);
        float xh[2][8], gx[2][8];
        float ab[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                xh[q][j] = (x[q][j] - mu[q]) * rs[q];
                gx[q][j] = g[q][j] * (1.0f + sc[j]);
                ab[2 * q] += gx[q][j];
                ab[2 * q + 1] += gx[q][j] * xh[q][j];
            }
        wg_sum<4>(ab, red, buf);
        buf ^= 1;
        if (live) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float dx[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    dx[j] = (gx[q][j] - ab[2 * q] * invC - xh[q][j] * ab[2 * q + 1] * invC) * rs[q];
                st16(dst[q], pack8(dx));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                part[0][j] += g[0][j] + g[1][j];
                part[1][j] += g[0][j] * xh[0][j] + g[1][j] * xh[1][j];
            }
        }
    }
    if (mod) {
        flush(cur);
        if (threadIdx.x == 0) leaf.cnt0[blockIdx.x] = n_ent;
    }
}

// ---------------------------------------------------------------------------
// modulate + RoPE backward in two kernels (C <= 3072)
// ---------------------------------------------------------------------------
// Kernel A, the per-token outputs, with the forward kernel's mapping: one
// wavefront per row (q or k) of a token, two tokens per workgroup; lane l
// owns the 16-byte chunks l, l+64, ... (all at in-head offset 8l mod D, so
// its four rotation angles serve every chunk); the row statistics are
// reductions inside the wavefront.  It writes dq, dk and each row's mean and
// 1/sigma (fp32).  Kernel B, the per-row sums: lane = one 8-channel chunk of
// a run of kSumRun tokens; it reads the rows again, turns dq', dk' back and
// normalises q, k with kernel A's statistics, and writes one entry per
// segment of equal adaLN row in the run; the segmented reduction then adds
// the entries.  Reading the four rows twice costs less than keeping 2 x 8
// fp32 sums per chunk in every wavefront, which does not fit two wavefronts
// per SIMD at C = 3072.
constexpr int kRowsTokens = 2;    // tokens per kernel-A workgroup

template <int NCH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NCH >= 6 ? 3 : 4))) void modrope_bwd_dx_kernel(
    ModRopeBwdArgs a, float* __restrict__ stats) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = int64_t(blockIdx.x) * kRowsTokens + (wave >> 1);
    const bool is_k = (wave & 1) != 0;
    if (t >= a.T) return;
    const int C = a.H * a.D;
    const int nch = C >> 3;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const bool mod = a.scale != nullptr;
    auto off = [&](int i) { return 16u * uint32_t(lane + kWave * i); };
    const __amdgpu_buffer_rsrc_t g_rs = make_rsrc((is_k ? a.dk_out : a.dq_out) + t * a.ld_gout, row_bytes);
    u32x4_t pg[NCH], px[NCH], usc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) pg[i] = bload16(g_rs, off(i), 0);
    if (mod) {
        const __amdgpu_buffer_rsrc_t x_rs = make_rsrc((is_k ? a.k_in : a.q_in) + t * a.ld_in, row_bytes);
        // a row outside [0, n_rows) reads zeros
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        const bool mok = m >= 0 && m < a.n_rows;
        const __amdgpu_buffer_rsrc_t sc_rs = make_rsrc(a.scale + int64_t(mok ? m : 0) * C, mok ? row_bytes : 0u);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            px[i] = bload16(x_rs, off(i), 0);
            usc[i] = bload16(sc_rs, off(i), 0);
        }
    }
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    float cs[4], sn[4];
    {
        const double p = double(a.pos[3 * t + axis]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = p * a.theta_turns[e0 / 2 + j];
            const float f = float(turns - rint(turns));
            sn[j] = __builtin_amdgcn_sinf(f);
            cs[j] = __builtin_amdgcn_cosf(f);
        }
    }
    // gradient with respect to the RoPE input: each pair turned back
    auto rot_back = [&](int i, float (&g)[8]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float h0 = bf_lo(pg[i][j]), h1 = bf_hi(pg[i][j]);
            g[2 * j] = h0 * cs[j] + h1 * sn[j];
            g[2 * j + 1] = -h0 * sn[j] + h1 * cs[j];
        }
    };
    const __amdgpu_buffer_rsrc_t d_rs = make_rsrc((is_k ? a.dk_in : a.dq_in) + t * a.ld_gin, row_bytes);
    if (!mod) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            float g[8];
            rot_back(i, g);
            bstore16(d_rs, off(i), 0, pack8(g));
        }
        return;
    }
    const float invC = 1.0f / float(C);
    // Register pins between the passes: the packed rows count as redefined
    // at each pin, so every pass widens them again instead of keeping the
    // widened fp32 copies live across the reductions.
    auto pin = [&] {
#pragma unroll
        for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(px[i]), "+v"(pg[i]), "+v"(usc[i]));
    };
    float sx = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) sx += bf_lo(px[i][w]) + bf_hi(px[i][w]);
    pin();
    const float mu = wave_sum(sx) * invC;
    float vx = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const bool inr = lane + kWave * i < nch;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float x0 = bf_lo(px[i][w]) - mu, x1 = bf_hi(px[i][w]) - mu;
            vx += inr ? x0 * x0 + x1 * x1 : 0.f;
        }
    }
    pin();
    const float rs = rsqrtf(wave_sum(vx) * invC + a.eps);
    // mean(gx) and mean(gx xh), gx = g (1 + scale); chunks past the row have g = 0
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float g[8], x[8], sc[8];
        rot_back(i, g);
        unpack8(px[i], x);
        unpack8(usc[i], sc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float gx = g[j] * (1.0f + sc[j]);
            sa += gx;
            sb += gx * ((x[j] - mu) * rs);
        }
    }
    pin();
    const float ma = wave_sum(sa) * invC, mb = wave_sum(sb) * invC;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        float g[8], x[8], sc[8], dx[8];
        rot_back(i, g);
        unpack8(px[i], x);
        unpack8(usc[i], sc);
#pragma unroll
        for (int j = 0; j < 8; ++j) dx[j] = (g[j] * (1.0f + sc[j]) - ma - (x[j] - mu) * rs * mb) * rs;
        bstore16(d_rs, off(i), 0, pack8(dx));
    }
    if (lane == 0) *reinterpret_cast<float2*>(stats + 4 * t + 2 * (is_k ? 1 : 0)) = float2{mu, rs};
}

// Kernel B: blockIdx.x = kRunsPerBlock runs of kSumRun tokens (one per
// wavefront), blockIdx.y = group of 64 chunks; lane = one chunk (in-head
// offset 8l mod D, as in kernel A).
__global__ __launch_bounds__(kWave * kRunsPerBlock) void modrope_bwd_sums_kernel(ModRopeBwdArgs a,
                                                                                const float* __restrict__ stats,
                                                                                SegLeaf leaf) {
    __shared__ int s_cnt[kRunsPerBlock];
    __shared__ int s_tag[kRunsPerBlock][kSumRun];
    zero_outputs(leaf);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t run = int64_t(blockIdx.x) * kRunsPerBlock + wave;
    const int C = a.H * a.D;
    const int nch = C >> 3;
    const int c = blockIdx.y * kWave + lane;
    const bool live = c < nch;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t voff = 16u * uint32_t(c);
    const int e0 = (8 * lane) % a.D;
    const int axis = e0 < a.rope_f ? 0 : (e0 < a.rope_f + a.rope_r ? 1 : 2);
    double th[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) th[j] = a.theta_turns[e0 / 2 + j];
    const int64_t t_begin = run * kSumRun;
    const int64_t t_end = t_begin + kSumRun < a.T ? t_begin + kSumRun : a.T;
    float sm[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sm[0][j] = sm[1][j] = 0.f;
    int cur = -1;
    int n_ent = 0;
    // the finished segment of row `row` becomes the run's next entry (rows
    // outside the table accumulate nothing)
    auto flush = [&](int row) {
        if (row < 0 || row >= a.n_rows) return;
        const int64_t pos = run * kSumRun + n_ent;
        put_entry<2>(sm, leaf.vals, pos, C, 8 * c, live);
        if (lane == 0) s_tag[wave][n_ent] = row;
        ++n_ent;
    };
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            flush(cur);
            cur = m;
        }
        const u32x4_t gq = bload16(make_rsrc(a.dq_out + t * a.ld_gout, row_bytes), voff, 0);
        const u32x4_t gk = bload16(make_rsrc(a.dk_out + t * a.ld_gout, row_bytes), voff, 0);
        const u32x4_t xq = bload16(make_rsrc(a.q_in + t * a.ld_in, row_bytes), voff, 0);
        const u32x4_t xk = bload16(make_rsrc(a.k_in + t * a.ld_in, row_bytes), voff, 0);
        const f32x4_t st = *reinterpret_cast<const f32x4_t*>(stats + 4 * t);   // mu_q, rs_q, mu_k, rs_k
        const double p = double(a.pos[3 * t + axis]);
        if (m < 0 || m >= a.n_rows) continue;   // a row outside the table adds nothing
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double turns = p * th[j];
            const float f = float(turns - rint(turns));
            const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
            const float q0 = bf_lo(gq[j]), q1 = bf_hi(gq[j]), k0 = bf_lo(gk[j]), k1 = bf_hi(gk[j]);
            const float gq0 = q0 * cs + q1 * sn, gq1 = -q0 * sn + q1 * cs;
            const float gk0 = k0 * cs + k1 * sn, gk1 = -k0 * sn + k1 * cs;
            const float hq0 = (bf_lo(xq[j]) - st[0]) * st[1], hq1 = (bf_hi(xq[j]) - st[0]) * st[1];
            const float hk0 = (bf_lo(xk[j]) - st[2]) * st[3], hk1 = (bf_hi(xk[j]) - st[2]) * st[3];
            sm[0][2 * j] += gq0 + gk0;
            sm[0][2 * j + 1] += gq1 + gk1;
            sm[1][2 * j] += gq0 * hq0 + gk0 * hk0;
            sm[1][2 * j + 1] += gq1 * hq1 + gk1 * hk1;
        }
    }
    flush(cur);
    if (lane == 0) s_cnt[wave] = n_ent;
    __syncthreads();   // the runs' entries are written (workgroup scope) and their rows are in LDS
    merge_block_runs<2>(leaf, s_cnt, s_tag, C);
}

int block_threads(int C) { return ((C / 8 + 63) / 64) * 64; }

// ---------------------------------------------------------------------------
// gated residual backward in two kernels
// ---------------------------------------------------------------------------
// Kernel A: one workgroup per token, one 16-byte chunk per thread (the
// forward kernel's mapping), LayerNorm reductions through LDS; it writes dx,
// do and, with the fused adaLN, the token's mean and 1/sigma of y and the
// means of g2 and g2 yh (g2 = dz (1 + scale2)).  Kernel B: lane = one
// 8-channel chunk of a run of kSumRun tokens; it recomputes dyt in fp32 from
// the rows and those statistics and writes the run's segment entries of
// dgate (and dshift2, dscale2), as the modulate + RoPE sums kernel does.
template <bool FUSED>
__global__ __launch_bounds__(1024) void gres_bwd_rows_kernel(GatedResBwdArgs a, float* __restrict__ stats) {
    __shared__ float red[2 * 2 * 16];
    const int64_t t = blockIdx.x;
    const int c = threadIdx.x;
    const int C = a.C;
    const bool in = c < (C >> 3);
    const int m0 = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
    const bool mok = m0 >= 0 && m0 < a.n_rows;      // a row outside the table reads zeros
    const int64_t m = mok ? m0 : 0;
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t mrow_bytes = mok ? row_bytes : 0u;
    const uint32_t off = 16u * uint32_t(c);
    float xv[8], ov[8], gv[8], dy[8], y[8];
    unpack8(bload16(make_rsrc(a.x + t * C, row_bytes), off, 0), xv);
    unpack8(bload16(make_rsrc(a.o + t * C, row_bytes), off, 0), ov);
    unpack8(bload16(make_rsrc(a.gate + m * C, mrow_bytes), off, 0), gv);
    unpack8(a.dy != nullptr ? bload16(make_rsrc(a.dy + t * C, row_bytes), off, 0) : u32x4_t{}, dy);
    u32x4_t pz = {0u, 0u, 0u, 0u}, ps2 = {0u, 0u, 0u, 0u};
    if constexpr (FUSED) {
        pz = bload16(make_rsrc(a.dz + t * C, row_bytes), off, 0);
        ps2 = bload16(make_rsrc(a.scale2 + m * C, mrow_bytes), off, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = xv[j] + gv[j] * ov[j];
    if constexpr (FUSED) {
        const float invC = 1.0f / float(C);
        float s[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) s[0] += y[j];        // chunks past the row hold y = 0
        wg_sum<2>(s, red, 0);
        const float mu = s[0] * invC;
        float v[2] = {0.f, 0.f};
        if (in)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[0] += (y[j] - mu) * (y[j] - mu);
        wg_sum<2>(v, red, 1);
        const float rs = rsqrtf(v[0] * invC + a.eps);
        float dz[8], s2[8], yh[8], g2[8];
        unpack8(pz, dz);
        unpack8(ps2, s2);
        float ab[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            yh[j] = (y[j] - mu) * rs;
            g2[j] = dz[j] * (1.0f + s2[j]);
            ab[0] += g2[j];
            ab[1] += g2[j] * yh[j];
        }
        wg_sum<2>(ab, red, 0);
        const float ma = ab[0] * invC, mb = ab[1] * invC;
#pragma unroll
        for (int j = 0; j < 8; ++j) dy[j] += (g2[j] - ma - yh[j] * mb) * rs;
        if (c == 0) *reinterpret_cast<f32x4_t*>(stats + 4 * t) = f32x4_t{mu, rs, ma, mb};
    }
    float dov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dov[j] = gv[j] * dy[j];
    bstore16(make_rsrc(a.dx + t * C, row_bytes), off, 0, pack8(dy));
    bstore16(make_rsrc(a.dout + t * C, row_bytes), off, 0, pack8(dov));
}

template <bool FUSED>
__global__ __launch_bounds__(kWave * kRunsPerBlock) void gres_bwd_sums_kernel(GatedResBwdArgs a,
                                                                             const float* __restrict__ stats,
                                                                             SegLeaf leaf) {
    __shared__ int s_cnt[kRunsPerBlock];
    __shared__ int s_tag[kRunsPerBlock][kSumRun];
    zero_outputs(leaf);
    constexpr int NA = FUSED ? 3 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t run = int64_t(blockIdx.x) * kRunsPerBlock + wave;
    const int C = a.C;
    const int c = blockIdx.y * kWave + lane;
    const bool live = c < (C >> 3);
    const uint32_t row_bytes = uint32_t(C) * 2u;
    const uint32_t voff = 16u * uint32_t(c);
    const int64_t t_begin = run * kSumRun;
    const int64_t t_end = t_begin + kSumRun < a.T ? t_begin + kSumRun : a.T;
    float sm[NA][8];
#pragma unroll
    for (int k = 0; k < NA; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) sm[k][j] = 0.f;
    int cur = -1;
    int n_ent = 0;
    float gv[8], s2[8];
    // the finished segment of row `row` becomes the run's next entry (rows
    // outside the table accumulate nothing)
    auto flush = [&](int row) {
        if (row < 0 || row >= a.n_rows) return;
        const int64_t pos = run * kSumRun + n_ent;
        put_entry<NA>(sm, leaf.vals, pos, C, 8 * c, live);
        if (lane == 0) s_tag[wave][n_ent] = row;
        ++n_ent;
    };
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int m = __builtin_amdgcn_readfirstlane(a.mod_row[t]);
        if (m != cur) {
            flush(cur);
            cur = m;
            const bool mok = m >= 0 && m < a.n_rows;
            const int64_t mm = mok ? m : 0;
            unpack8(bload16(make_rsrc(a.gate + mm * C, mok ? row_bytes : 0u), voff, 0), gv);
            if constexpr (FUSED) unpack8(bload16(make_rsrc(a.scale2 + mm * C, mok ? row_bytes : 0u), voff, 0), s2);
        }
        float xv[8], ov[8], dy[8], dz[8];
        unpack8(bload16(make_rsrc(a.x + t * C, row_bytes), voff, 0), xv);
        unpack8(bload16(make_rsrc(a.o + t * C, row_bytes), voff, 0), ov);
        unpack8(a.dy != nullptr ? bload16(make_rsrc(a.dy + t * C, row_bytes), voff, 0) : u32x4_t{}, dy);
        f32x4_t st = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FUSED) {
            unpack8(bload16(make_rsrc(a.dz + t * C, row_bytes), voff, 0), dz);
            st = *reinterpret_cast<const f32x4_t*>(stats + 4 * t);   // mu, rs, mean g2, mean g2 yh
        }
        if (m < 0 || m >= a.n_rows) continue;    // a row outside the table adds nothing
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float dyt = dy[j];
            if constexpr (FUSED) {
                const float yh = (xv[j] + gv[j] * ov[j] - st[0]) * st[1];
                dyt += (dz[j] * (1.0f + s2[j]) - st[2] - yh * st[3]) * st[1];
                sm[1][j] += dz[j];
                sm[2][j] += dz[j] * yh;
            }
            sm[0][j] += dyt * ov[j];
        }
    }
    flush(cur);
    if (lane == 0) s_cnt[wave] = n_ent;
    __syncthreads();   // the runs' entries are written (workgroup scope) and their rows are in LDS
    merge_block_runs<NA>(leaf, s_cnt, s_tag, C);
}

}  // namespace

size_t elementwise_bwd_workspace_bytes(int64_t T, int32_t C, int32_t n_arrays) {
    const int64_t Tn = T < 0 ? 0 : T;
    if (Tn == 0 || C <= 0 || n_arrays <= 0) return 0;
    // entries of runs of kRun (the single-kernel form) or kLeafSpan tokens,
    // the reduction's tags and counts, and 16 bytes of statistics per token
    const size_t a = seg_layout(Tn, C, n_arrays, kRun).total;
    const size_t b = seg_layout(Tn, C, n_arrays, kLeafSpan).total;
    return a > b ? a : b;
}

hipError_t launch_modulate_rope_bwd(const ModRopeBwdArgs& args, hipStream_t stream) {
    ModRopeBwdArgs a = args;
    const int dims[3] = {a.rope_f, a.rope_r, a.rope_c};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
        for (int j = 0; j < dims[ax] / 2; ++j)
            a.theta_turns[pair++] = std::pow(double(a.rope_base), -2.0 * j / double(dims[ax])) *
                                    0.15915494309189535;   // radians -> turns (1 / 2 pi)
    const int C = a.H * a.D;
    const bool mod = a.scale != nullptr;
    if (a.T == 0)   // no tokens: the row sums are zero (otherwise the reduction's last level writes every row)
        return mod ? zero_f32(a.dshift, a.dscale, nullptr, int64_t(a.n_rows) * C, stream) : hipSuccess;
    const int nch_w = (C / 8 + kWave - 1) / kWave;     // 16-byte chunks per lane of a row
    if (nch_w > 6) {
        const SegLayout L = seg_layout(a.T, C, 2, kRun);
        hipLaunchKernelGGL(modulate_rope_bwd_kernel, dim3(unsigned(L.n_runs)), dim3(block_threads(C)), 0, stream, a,
                           seg_leaf(L, a.workspace, a.n_rows, a.dshift, a.dscale, nullptr));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !mod) return e;
        return reduce_segments<2>(L, a.workspace, a.n_rows, a.dshift, a.dscale, nullptr, stream);
    }
    // two kernels: the rows' statistics and the entries in the workspace
    const SegLayout L = seg_layout(a.T, C, 2, kLeafSpan);
    float* stats = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + L.off_stats);
    const dim3 grid_a(unsigned((a.T + kRowsTokens - 1) / kRowsTokens));
    switch (nch_w) {
        case 1: hipLaunchKernelGGL(modrope_bwd_dx_kernel<1>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 2: hipLaunchKernelGGL(modrope_bwd_dx_kernel<2>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 3: hipLaunchKernelGGL(modrope_bwd_dx_kernel<3>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 4: hipLaunchKernelGGL(modrope_bwd_dx_kernel<4>, grid_a, dim3(256), 0, stream, a, stats); break;
        case 5: hipLaunchKernelGGL(modrope_bwd_dx_kernel<5>, grid_a, dim3(256), 0, stream, a, stats); break;
        default: hipLaunchKernelGGL(modrope_bwd_dx_kernel<6>, grid_a, dim3(256), 0, stream, a, stats); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !mod) return e;
    hipLaunchKernelGGL(modrope_bwd_sums_kernel, dim3(unsigned(L.n_runs), unsigned((C / 8 + kWave - 1) / kWave)),
                       dim3(kWave * kRunsPerBlock), 0, stream, a, stats,
                       seg_leaf(L, a.workspace, a.n_rows, a.dshift, a.dscale, nullptr));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return reduce_segments<2>(L, a.workspace, a.n_rows, a.dshift, a.dscale, nullptr, stream);
}

hipError_t launch_gated_residual_bwd(const GatedResBwdArgs& a, hipStream_t stream) {
    const bool fused = a.dz != nullptr;
    if (a.T == 0)   // no tokens: the row sums are zero (otherwise the reduction's last level writes every row)
        return zero_f32(a.dgate, fused ? a.dshift2 : nullptr, fused ? a.dscale2 : nullptr, int64_t(a.n_rows) * a.C,
                        stream);
    hipError_t e = hipSuccess;
    // the rows' statistics and the runs' entries (1 or 3 arrays) in the
    // workspace; it fits the size the query returns (sized for 3 arrays)
    const int na = fused ? 3 : 1;
    const SegLayout L = seg_layout(a.T, a.C, na, kLeafSpan);
    float* stats = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + L.off_stats);
    const SegLeaf leaf = seg_leaf(L, a.workspace, a.n_rows, a.dgate, fused ? a.dshift2 : nullptr,
                                  fused ? a.dscale2 : nullptr);
    const dim3 grid_b(unsigned(L.n_runs), unsigned((a.C / 8 + kWave - 1) / kWave));
    if (fused) {
        hipLaunchKernelGGL(gres_bwd_rows_kernel<true>, dim3(unsigned(a.T)), dim3(block_threads(a.C)), 0, stream, a,
                           stats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(gres_bwd_sums_kernel<true>, grid_b, dim3(kWave * kRunsPerBlock), 0, stream, a, stats,
                           leaf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return reduce_segments<3>(L, a.workspace, a.n_rows, a.dgate, a.dshift2, a.dscale2, stream);
    }
    hipLaunchKernelGGL(gres_bwd_rows_kernel<false>, dim3(unsigned(a.T)), dim3(block_threads(a.C)), 0, stream, a,
                       stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gres_bwd_sums_kernel<false>, grid_b, dim3(kWave * kRunsPerBlock), 0, stream, a, stats,
                       leaf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return reduce_segments<1>(L, a.workspace, a.n_rows, a.dgate, nullptr, nullptr, stream);
}

}  // namespace mf
