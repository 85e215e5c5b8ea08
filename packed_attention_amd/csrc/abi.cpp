// C-ABI entry points of libmf.so: argument validation on the host, optional
// table checks (MF_DEBUG=1), and launches on the caller's stream.  Every
// check runs before the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mf.h"
#include "mf_internal.h"

namespace mf {

int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

}  // namespace mf

namespace {

bool debug_mode() {
    static const bool on = [] {
        const char* e = std::getenv("MF_DEBUG");
        return e != nullptr && std::strcmp(e, "1") == 0;
    }();
    return on;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Arguments a workspace-size query can size: anything its call would reject
// for its sizes gets 0 bytes (and no arithmetic on out-of-range values).
inline bool query_ok(int64_t T, int32_t H, int32_t D) {
    return T >= 0 && T <= INT32_MAX && H > 0 && H <= 4096 && D > 0 && D <= 65536 && int64_t(H) * D <= 65536;
}

// Largest token stride (elements) any entry point takes: with T <= 2^31 every
// offset T * stride * element size then fits in 64 bits.
constexpr int64_t kMaxStride = int64_t(1) << 31;

inline mf_status from_hip(hipError_t e) { return e == hipSuccess ? MF_OK : MF_ERR_HIP; }

// Copy a device int32 array to the host (debug checks only).
bool fetch(const int32_t* dev, size_t n, std::vector<int32_t>& out, hipStream_t stream) {
    out.resize(n);
    if (n == 0) return true;
    if (hipStreamSynchronize(stream) != hipSuccess) return false;
    return hipMemcpy(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess;
}

// An adaLN table read by a forward call: at least one row when there are
// tokens, and every element offset below 2^31.
bool rows_ok(int32_t n_rows, int64_t T, int64_t C) {
    return n_rows >= (T > 0 ? 1 : 0) && int64_t(n_rows) * C <= (int64_t(1) << 31);
}

mf_status check_rows(const int32_t* mod_row, int64_t T, int32_t n_rows, hipStream_t stream) {
    std::vector<int32_t> h;
    if (!fetch(mod_row, size_t(T), h, stream)) return MF_ERR_HIP;
    for (int32_t m : h)
        if (m < 0 || m >= n_rows) return MF_ERR_TABLE;
    return MF_OK;
}

mf_status finish(hipError_t e, hipStream_t stream) {
    if (e != hipSuccess) return MF_ERR_HIP;
    if (debug_mode()) return from_hip(hipStreamSynchronize(stream));
    return MF_OK;
}

}  // namespace

extern "C" {

const char* mf_status_string(mf_status s) {
    switch (s) {
        case MF_OK: return "MF_OK";
        case MF_ERR_NULL: return "MF_ERR_NULL: a required pointer is NULL";
        case MF_ERR_SHAPE: return "MF_ERR_SHAPE: sizes, strides or rope dims out of range";
        case MF_ERR_ALIGN: return "MF_ERR_ALIGN: pointer or stride misaligned";
        case MF_ERR_UNSUPPORTED: return "MF_ERR_UNSUPPORTED: configuration not implemented";
        case MF_ERR_WORKSPACE: return "MF_ERR_WORKSPACE: workspace missing or too small";
        case MF_ERR_TABLE: return "MF_ERR_TABLE: invalid table contents";
        case MF_ERR_HIP: return "MF_ERR_HIP: the HIP runtime reported an error";
        default: return "MF_ERR_UNKNOWN";
    }
}

int32_t mf_abi_version(void) { return MF_ABI_VERSION; }

mf_status mf_modulate_rope(void* stream, const void* q_in, const void* k_in, void* q_out, void* k_out,
                           int64_t T, int32_t H, int32_t D, int64_t ld_in, int64_t ld_out,
                           const void* shift, const void* scale, const int32_t* mod_row, int32_t n_rows,
                           const int32_t* pos, int32_t rope_f, int32_t rope_r, int32_t rope_c,
                           float rope_base, float eps) {
    if (T < 0 || T > INT32_MAX || H <= 0) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (int64_t(H) * D > 8192) return MF_ERR_UNSUPPORTED;
    if (rope_f < 0 || rope_r < 0 || rope_c < 0 || rope_f % 8 || rope_r % 8 || rope_c % 8 ||
        rope_f + rope_r + rope_c != D)
        return MF_ERR_SHAPE;
    if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return MF_ERR_SHAPE;
    if (ld_in < int64_t(H) * D || ld_out < int64_t(H) * D) return MF_ERR_SHAPE;
    if (ld_in > kMaxStride || ld_out > kMaxStride) return MF_ERR_UNSUPPORTED;
    if ((shift == nullptr) != (scale == nullptr)) return MF_ERR_NULL;
    const bool modulate = shift != nullptr;
    if (modulate && !(eps > 0.f)) return MF_ERR_SHAPE;
    if (modulate && !rows_ok(n_rows, T, int64_t(H) * D)) return MF_ERR_SHAPE;
    if (T == 0) return MF_OK;
    if (!q_in || !k_in || !q_out || !k_out || !pos) return MF_ERR_NULL;
    if (modulate && !mod_row) return MF_ERR_NULL;
    if (ld_in % 8 || ld_out % 8) return MF_ERR_ALIGN;
    if (!aligned(q_in, 16) || !aligned(k_in, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
        !aligned(pos, 4))
        return MF_ERR_ALIGN;
    if (modulate && (!aligned(shift, 16) || !aligned(scale, 16) || !aligned(mod_row, 4)))
        return MF_ERR_ALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> hp;
        if (!fetch(pos, size_t(T) * 3, hp, s)) return MF_ERR_HIP;
        for (int32_t v : hp)
            if (v < 0) return MF_ERR_TABLE;
        if (modulate) {
            mf_status st = check_rows(mod_row, T, n_rows, s);
            if (st != MF_OK) return st;
        }
    }
    mf::ModRopeArgs a;
    a.q_in = static_cast<const uint16_t*>(q_in);
    a.k_in = static_cast<const uint16_t*>(k_in);
    a.q_out = static_cast<uint16_t*>(q_out);
    a.k_out = static_cast<uint16_t*>(k_out);
    a.T = T; a.H = H; a.D = D; a.ld_in = ld_in; a.ld_out = ld_out;
    a.shift = static_cast<const uint16_t*>(shift);
    a.scale = static_cast<const uint16_t*>(scale);
    a.mod_row = mod_row; a.n_rows = modulate ? n_rows : 0; a.pos = pos;
    a.rope_f = rope_f; a.rope_r = rope_r; a.rope_c = rope_c;
    a.rope_base = rope_base; a.eps = eps;
    return finish(mf::launch_modulate_rope(a, s), s);
}

size_t mf_varlen_attn_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D) {
    if (!query_ok(T, H, D) || n_seq < 0 || n_seq > (1 << 24)) return 0;
    return mf::attn_workspace_bytes(n_seq, T, H, D);
}

}  // extern "C"

namespace {

// Argument checks shared by the two forward-attention entry points (all on
// the host, before any HIP call); fills the launch arguments.
mf_status attn_fwd_args(void* stream, const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen, int64_t T, int32_t H,
                        int32_t D, int64_t ld_qkv, int64_t ld_o, float softmax_scale, mf::AttnArgs& a) {
    if (T < 0 || T > INT32_MAX || H <= 0 || H > 4096) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (n_seq < 0 || (T > 0 && n_seq < 1) || n_seq > (1 << 24)) return MF_ERR_SHAPE;
    if (max_seqlen < 0 || max_seqlen > T || (T > 0 && max_seqlen == 0)) return MF_ERR_SHAPE;
    if (ld_qkv < int64_t(H) * D || ld_o < int64_t(H) * D) return MF_ERR_SHAPE;
    if (ld_qkv > kMaxStride || ld_o > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MF_ERR_SHAPE;
    // 32-bit buffer offsets inside one sequence's rows (plus a ragged tile)
    if ((int64_t(max_seqlen) + 256) * ld_qkv * 2 >= (int64_t(1) << 32)) return MF_ERR_UNSUPPORTED;
    // work units must fit a 1D grid
    if (int64_t(H) * (T / 128 + 1 + n_seq) > (int64_t(1) << 30)) return MF_ERR_SHAPE;
    if (T > 0) {
        if (!q || !k || !v || !o || !cu_seqlens) return MF_ERR_NULL;
        if (ld_qkv % 8 || ld_o % 8) return MF_ERR_ALIGN;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(cu_seqlens, 4) || (lse && !aligned(lse, 4)))
            return MF_ERR_ALIGN;
    }
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse; a.cu_seqlens = cu_seqlens; a.n_seq = n_seq; a.max_seqlen = max_seqlen;
    a.T = T; a.H = H; a.D = D; a.ld_qkv = ld_qkv; a.ld_o = ld_o;
    a.softmax_scale = softmax_scale; a.workspace = nullptr; a.workspace_bytes = 0;
    (void)stream;
    return MF_OK;
}

// MF_DEBUG table checks of the forward attention.
mf_status attn_fwd_debug_tables(const mf::AttnArgs& a, hipStream_t s) {
    std::vector<int32_t> cu;
    if (!fetch(a.cu_seqlens, size_t(a.n_seq) + 1, cu, s)) return MF_ERR_HIP;
    if (cu[0] != 0 || cu[a.n_seq] != a.T) return MF_ERR_TABLE;
    for (int32_t i = 0; i < a.n_seq; ++i) {
        const int64_t L = int64_t(cu[i + 1]) - cu[i];
        if (L < 0 || L > a.max_seqlen) return MF_ERR_TABLE;
    }
    return MF_OK;
}

}  // namespace

extern "C" {

mf_status mf_varlen_attn_fwd(void* stream, const void* q, const void* k, const void* v, void* o,
                             float* lse, const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen,
                             int64_t T, int32_t H, int32_t D, int64_t ld_qkv, int64_t ld_o,
                             float softmax_scale, void* workspace, size_t workspace_bytes) {
    mf::AttnArgs a;
    mf_status st = attn_fwd_args(stream, q, k, v, o, lse, cu_seqlens, n_seq, max_seqlen, T, H, D, ld_qkv,
                                 ld_o, softmax_scale, a);
    if (st != MF_OK) return st;
    if (T == 0) return MF_OK;
    const size_t need = mf::attn_workspace_bytes(n_seq, T, H, D);
    if (workspace == nullptr || workspace_bytes < need) return MF_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        st = attn_fwd_debug_tables(a, s);
        if (st != MF_OK) return st;
    }
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return finish(mf::launch_varlen_attn_fwd(a, s), s);
}

mf_status mf_varlen_attn_fwd_noalloc(void* stream, const void* q, const void* k, const void* v, void* o,
                                     float* lse, const int32_t* cu_seqlens, int32_t n_seq,
                                     int32_t max_seqlen, int64_t T, int32_t H, int32_t D, int64_t ld_qkv,
                                     int64_t ld_o, float softmax_scale) {
    mf::AttnArgs a;
    mf_status st = attn_fwd_args(stream, q, k, v, o, lse, cu_seqlens, n_seq, max_seqlen, T, H, D, ld_qkv,
                                 ld_o, softmax_scale, a);
    if (st != MF_OK) return st;
    if (T == 0) return MF_OK;
    if (mf::attn_workspace_bytes(n_seq, T, H, D) > mf::kAttnNoAllocScratchBytes) return MF_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        st = attn_fwd_debug_tables(a, s);
        if (st != MF_OK) return st;
    }
    return finish(mf::launch_varlen_attn_fwd_noalloc(a, s), s);
}

mf_status mf_set_attn_fwd_grid(int32_t g) {
    if (g < 0 || g > 65536) return MF_ERR_SHAPE;
    mf::set_attn_fwd_grid(g);
    return MF_OK;
}

size_t mf_varlen_attn_bwd_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D) {
    if (!query_ok(T, H, D) || n_seq < 0 || n_seq > (1 << 24)) return 0;
    return mf::attn_bwd_workspace_bytes(n_seq, T, H, D);
}

mf_status mf_varlen_attn_bwd(void* stream, const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens, int32_t n_seq, int32_t max_seqlen, int64_t T,
                             int32_t H, int32_t D, int64_t ld_qkv, int64_t ld_o, int64_t ld_dqkv,
                             float softmax_scale, void* workspace, size_t workspace_bytes) {
    if (T < 0 || T > INT32_MAX || H <= 0 || H > 4096) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (n_seq < 0 || (T > 0 && n_seq < 1) || n_seq > (1 << 24)) return MF_ERR_SHAPE;
    if (max_seqlen < 0 || max_seqlen > T || (T > 0 && max_seqlen == 0)) return MF_ERR_SHAPE;
    if (ld_qkv < int64_t(H) * D || ld_o < int64_t(H) * D || ld_dqkv < int64_t(H) * D) return MF_ERR_SHAPE;
    if (ld_qkv > kMaxStride || ld_o > kMaxStride || ld_dqkv > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MF_ERR_SHAPE;
    // 32-bit buffer offsets inside one sequence's rows (plus a ragged tile)
    const int64_t ld_max = ld_qkv > ld_o ? ld_qkv : ld_o;
    if ((int64_t(max_seqlen) + 256) * ld_max * 2 >= (int64_t(1) << 32)) return MF_ERR_UNSUPPORTED;
    // work units must fit a 1D grid
    if (int64_t(H) * (T / 128 + 1 + n_seq) > (int64_t(1) << 30)) return MF_ERR_SHAPE;
    if (T == 0) return MF_OK;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens) return MF_ERR_NULL;
    if (ld_qkv % 8 || ld_o % 8 || ld_dqkv % 8) return MF_ERR_ALIGN;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) ||
        !aligned(cu_seqlens, 4))
        return MF_ERR_ALIGN;
    const size_t need = mf::attn_bwd_workspace_bytes(n_seq, T, H, D);
    if (workspace == nullptr || workspace_bytes < need) return MF_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MF_ERR_ALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> cu;
        if (!fetch(cu_seqlens, size_t(n_seq) + 1, cu, s)) return MF_ERR_HIP;
        if (cu[0] != 0 || cu[n_seq] != T) return MF_ERR_TABLE;
        for (int32_t i = 0; i < n_seq; ++i) {
            const int64_t L = int64_t(cu[i + 1]) - cu[i];
            if (L < 0 || L > max_seqlen) return MF_ERR_TABLE;
        }
    }
    mf::AttnBwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<const uint16_t*>(o);
    a.dout = static_cast<const uint16_t*>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.cu_seqlens = cu_seqlens; a.n_seq = n_seq; a.max_seqlen = max_seqlen;
    a.T = T; a.H = H; a.D = D; a.ld_qkv = ld_qkv; a.ld_o = ld_o; a.ld_d = ld_dqkv;
    a.softmax_scale = softmax_scale; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return finish(mf::launch_varlen_attn_bwd(a, s), s);
}

mf_status mf_gated_residual(void* stream, const void* x, const void* o, void* y, const void* gate,
                            const int32_t* mod_row, int32_t n_rows, const void* shift2, const void* scale2,
                            void* z, int64_t T, int32_t C, float eps) {
    if (T < 0 || T > INT32_MAX || C <= 0 || C % 64 || C > 8192) return MF_ERR_SHAPE;
    if (!rows_ok(n_rows, T, C)) return MF_ERR_SHAPE;
    const int n_fused = (shift2 != nullptr) + (scale2 != nullptr) + (z != nullptr);
    if (n_fused != 0 && n_fused != 3) return MF_ERR_NULL;
    if (n_fused == 3 && !(eps > 0.f)) return MF_ERR_SHAPE;
    if (T == 0) return MF_OK;
    if (!x || !o || !y || !gate || !mod_row) return MF_ERR_NULL;
    if (!aligned(x, 16) || !aligned(o, 16) || !aligned(y, 16) || !aligned(gate, 16) ||
        !aligned(mod_row, 4))
        return MF_ERR_ALIGN;
    if (n_fused == 3 && (!aligned(shift2, 16) || !aligned(scale2, 16) || !aligned(z, 16)))
        return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        mf_status st = check_rows(mod_row, T, n_rows, s);
        if (st != MF_OK) return st;
    }
    mf::GatedResArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.o = static_cast<const uint16_t*>(o);
    a.y = static_cast<uint16_t*>(y);
    a.gate = static_cast<const uint16_t*>(gate);
    a.mod_row = mod_row;
    a.n_rows = n_rows;
    a.shift2 = static_cast<const uint16_t*>(shift2);
    a.scale2 = static_cast<const uint16_t*>(scale2);
    a.z = static_cast<uint16_t*>(z);
    a.T = T; a.C = C; a.eps = eps;
    return finish(mf::launch_gated_residual(a, s), s);
}

size_t mf_modulate_rope_bwd_workspace_bytes(int64_t T, int32_t H, int32_t D) {
    if (!query_ok(T, H, D)) return 0;
    return mf::elementwise_bwd_workspace_bytes(T, H * D, 2);
}

size_t mf_gated_residual_bwd_workspace_bytes(int64_t T, int32_t C) {
    if (!query_ok(T, 1, C)) return 0;
    return mf::elementwise_bwd_workspace_bytes(T, C, 3);
}

mf_status mf_modulate_rope_bwd(void* stream, const void* q_in, const void* k_in, int64_t ld_in,
                               const void* dq_out, const void* dk_out, int64_t ld_gout, void* dq_in,
                               void* dk_in, int64_t ld_gin, int64_t T, int32_t H, int32_t D,
                               const void* scale, const int32_t* mod_row, int32_t n_rows, float* dshift,
                               float* dscale, const int32_t* pos, int32_t rope_f, int32_t rope_r,
                               int32_t rope_c, float rope_base, float eps, void* workspace,
                               size_t workspace_bytes) {
    if (T < 0 || T > INT32_MAX || H <= 0) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (int64_t(H) * D > 8192) return MF_ERR_UNSUPPORTED;
    if (rope_f < 0 || rope_r < 0 || rope_c < 0 || rope_f % 8 || rope_r % 8 || rope_c % 8 ||
        rope_f + rope_r + rope_c != D)
        return MF_ERR_SHAPE;
    if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return MF_ERR_SHAPE;
    if (ld_in < int64_t(H) * D || ld_gout < int64_t(H) * D || ld_gin < int64_t(H) * D) return MF_ERR_SHAPE;
    if (ld_in > kMaxStride || ld_gout > kMaxStride || ld_gin > kMaxStride) return MF_ERR_UNSUPPORTED;
    const bool modulate = scale != nullptr;
    if (modulate && (!(eps > 0.f) || n_rows <= 0)) return MF_ERR_SHAPE;
    if (modulate && int64_t(n_rows) * H * D > (int64_t(1) << 31)) return MF_ERR_SHAPE;
    if (T == 0) {
        // nothing to read; the row sums are still defined (zero)
        if (!modulate) return MF_OK;
        if (!dshift || !dscale) return MF_ERR_NULL;
    } else {
        if (!q_in || !k_in || !dq_out || !dk_out || !dq_in || !dk_in || !pos) return MF_ERR_NULL;
        if (modulate && (!mod_row || !dshift || !dscale)) return MF_ERR_NULL;
        if (ld_in % 8 || ld_gout % 8 || ld_gin % 8) return MF_ERR_ALIGN;
        if (!aligned(q_in, 16) || !aligned(k_in, 16) || !aligned(dq_out, 16) || !aligned(dk_out, 16) ||
            !aligned(dq_in, 16) || !aligned(dk_in, 16) || !aligned(pos, 4))
            return MF_ERR_ALIGN;
    }
    if (modulate && (!aligned(scale, 16) || !aligned(dshift, 4) || !aligned(dscale, 4) ||
                     (T > 0 && !aligned(mod_row, 4))))
        return MF_ERR_ALIGN;
    if (modulate && T > 0) {
        if (workspace == nullptr || workspace_bytes < mf::elementwise_bwd_workspace_bytes(T, H * D, 2))
            return MF_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return MF_ERR_ALIGN;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode() && T > 0) {
        std::vector<int32_t> hp;
        if (!fetch(pos, size_t(T) * 3, hp, s)) return MF_ERR_HIP;
        for (int32_t v : hp)
            if (v < 0) return MF_ERR_TABLE;
        if (modulate) {
            std::vector<int32_t> hm;
            if (!fetch(mod_row, size_t(T), hm, s)) return MF_ERR_HIP;
            for (int32_t m : hm)
                if (m < 0 || m >= n_rows) return MF_ERR_TABLE;
        }
    }
    mf::ModRopeBwdArgs a;
    a.q_in = static_cast<const uint16_t*>(q_in);
    a.k_in = static_cast<const uint16_t*>(k_in);
    a.dq_out = static_cast<const uint16_t*>(dq_out);
    a.dk_out = static_cast<const uint16_t*>(dk_out);
    a.dq_in = static_cast<uint16_t*>(dq_in);
    a.dk_in = static_cast<uint16_t*>(dk_in);
    a.T = T; a.H = H; a.D = D; a.ld_in = ld_in; a.ld_gout = ld_gout; a.ld_gin = ld_gin;
    a.scale = static_cast<const uint16_t*>(scale);
    a.mod_row = mod_row; a.n_rows = n_rows; a.dshift = dshift; a.dscale = dscale; a.pos = pos;
    a.rope_f = rope_f; a.rope_r = rope_r; a.rope_c = rope_c; a.rope_base = rope_base; a.eps = eps;
    a.workspace = workspace;
    return finish(mf::launch_modulate_rope_bwd(a, s), s);
}

mf_status mf_gated_residual_bwd(void* stream, const void* x, const void* o, const void* gate,
                                const int32_t* mod_row, int32_t n_rows, const void* dy, const void* scale2,
                                const void* dz, void* dx, void* dout, float* dgate, float* dshift2,
                                float* dscale2, int64_t T, int32_t C, float eps, void* workspace,
                                size_t workspace_bytes) {
    if (T < 0 || T > INT32_MAX || C <= 0 || C % 64 || C > 8192) return MF_ERR_SHAPE;
    if (n_rows <= 0 || int64_t(n_rows) * C > (int64_t(1) << 31)) return MF_ERR_SHAPE;
    const int n_fused = (scale2 != nullptr) + (dz != nullptr) + (dshift2 != nullptr) + (dscale2 != nullptr);
    if (n_fused != 0 && n_fused != 4) return MF_ERR_NULL;
    const bool fused = n_fused == 4;
    if (fused && !(eps > 0.f)) return MF_ERR_SHAPE;
    if (!dgate) return MF_ERR_NULL;
    if (T > 0 && (!x || !o || !gate || !mod_row || !dx || !dout)) return MF_ERR_NULL;
    if (!aligned(dgate, 4) || (fused && (!aligned(dshift2, 4) || !aligned(dscale2, 4))))
        return MF_ERR_ALIGN;
    if (T > 0) {
        if (!aligned(x, 16) || !aligned(o, 16) || !aligned(gate, 16) || !aligned(mod_row, 4) ||
            !aligned(dx, 16) || !aligned(dout, 16) || (dy && !aligned(dy, 16)))
            return MF_ERR_ALIGN;
        if (fused && (!aligned(scale2, 16) || !aligned(dz, 16))) return MF_ERR_ALIGN;
        if (workspace == nullptr || workspace_bytes < mf::elementwise_bwd_workspace_bytes(T, C, fused ? 3 : 1))
            return MF_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return MF_ERR_ALIGN;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode() && T > 0) {
        std::vector<int32_t> hm;
        if (!fetch(mod_row, size_t(T), hm, s)) return MF_ERR_HIP;
        for (int32_t m : hm)
            if (m < 0 || m >= n_rows) return MF_ERR_TABLE;
    }
    mf::GatedResBwdArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.o = static_cast<const uint16_t*>(o);
    a.gate = static_cast<const uint16_t*>(gate);
    a.mod_row = mod_row; a.n_rows = n_rows;
    a.dy = static_cast<const uint16_t*>(dy);
    a.scale2 = static_cast<const uint16_t*>(scale2);
    a.dz = static_cast<const uint16_t*>(dz);
    a.dx = static_cast<uint16_t*>(dx);
    a.dout = static_cast<uint16_t*>(dout);
    a.dgate = dgate; a.dshift2 = dshift2; a.dscale2 = dscale2;
    a.T = T; a.C = C; a.eps = eps; a.workspace = workspace;
    return finish(mf::launch_gated_residual_bwd(a, s), s);
}

size_t mf_block_qkv_workspace_bytes(int64_t T, int32_t H, int32_t D) {
    if (!query_ok(T, H, D)) return 0;
    return mf::block_qkv_workspace_bytes(T, H * D, D);
}

mf_status mf_block_qkv(void* stream, const void* x, int64_t ld_x, const void* w_qkv, void* qkv,
                       int64_t ld_qkv, const void* shift, const void* scale, const int32_t* mod_row,
                       int32_t n_rows, const int32_t* pos, int64_t T, int32_t H, int32_t D, int32_t rope_f, int32_t rope_r,
                       int32_t rope_c, float rope_base, float eps, void* workspace, size_t workspace_bytes) {
    if (T < 0 || T > INT32_MAX || H <= 0) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    const int64_t C = int64_t(H) * D;
    if (C > 8192) return MF_ERR_UNSUPPORTED;
    if (rope_f < 0 || rope_r < 0 || rope_c < 0 || rope_f % 8 || rope_r % 8 || rope_c % 8 ||
        rope_f + rope_r + rope_c != D)
        return MF_ERR_SHAPE;
    if (!(rope_base > 0.f) || !std::isfinite(rope_base)) return MF_ERR_SHAPE;
    if (ld_x < C || ld_qkv < 3 * C) return MF_ERR_SHAPE;
    if (ld_x > kMaxStride || ld_qkv > kMaxStride) return MF_ERR_UNSUPPORTED;
    // 32-bit buffer offsets over the activations and the weights
    if (T * ld_x * 2 >= (int64_t(1) << 32) || 3 * C * C * 2 >= (int64_t(1) << 32)) return MF_ERR_UNSUPPORTED;
    if ((shift == nullptr) != (scale == nullptr)) return MF_ERR_NULL;
    const bool modulate = shift != nullptr;
    if (modulate && !(eps > 0.f)) return MF_ERR_SHAPE;
    if (modulate && !rows_ok(n_rows, T, C)) return MF_ERR_SHAPE;
    if (T == 0) return MF_OK;
    if (!x || !w_qkv || !qkv || !pos) return MF_ERR_NULL;
    if (modulate && !mod_row) return MF_ERR_NULL;
    if (ld_x % 8 || ld_qkv % 8) return MF_ERR_ALIGN;
    if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(qkv, 16) || !aligned(pos, 4)) return MF_ERR_ALIGN;
    if (modulate && (!aligned(shift, 16) || !aligned(scale, 16) || !aligned(mod_row, 4))) return MF_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < mf::block_qkv_workspace_bytes(T, int32_t(C), D))
        return MF_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> hp;
        if (!fetch(pos, size_t(T) * 3, hp, s)) return MF_ERR_HIP;
        for (int32_t v : hp)
            if (v < 0) return MF_ERR_TABLE;
        if (modulate) {
            mf_status st = check_rows(mod_row, T, n_rows, s);
            if (st != MF_OK) return st;
        }
    }
    mf::BlockQkvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.ld_x = ld_x;
    a.w = static_cast<const uint16_t*>(w_qkv);
    a.qkv = static_cast<uint16_t*>(qkv);
    a.ld_qkv = ld_qkv;
    a.shift = static_cast<const uint16_t*>(shift);
    a.scale = static_cast<const uint16_t*>(scale);
    a.mod_row = mod_row; a.n_rows = modulate ? n_rows : 0; a.pos = pos;
    a.T = T; a.H = H; a.D = D;
    a.rope_f = rope_f; a.rope_r = rope_r; a.rope_c = rope_c;
    a.rope_base = rope_base; a.eps = eps;
    a.workspace = workspace;
    return finish(mf::launch_block_qkv(a, s), s);
}

mf_status mf_block_out(void* stream, const void* o, int64_t ld_o, const void* w_o, const void* x,
                       const void* gate, const int32_t* mod_row, int32_t n_rows, void* y, int64_t T, int32_t C) {
    if (T < 0 || T > INT32_MAX || C <= 0 || C % 64 || C > 8192) return MF_ERR_SHAPE;
    if (!rows_ok(n_rows, T, C)) return MF_ERR_SHAPE;
    if (ld_o < C) return MF_ERR_SHAPE;
    if (ld_o > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (T * ld_o * 2 >= (int64_t(1) << 32)) return MF_ERR_UNSUPPORTED;
    if (T == 0) return MF_OK;
    if (!o || !w_o || !x || !gate || !mod_row || !y) return MF_ERR_NULL;
    if (ld_o % 8) return MF_ERR_ALIGN;
    if (!aligned(o, 16) || !aligned(w_o, 16) || !aligned(x, 16) || !aligned(gate, 16) || !aligned(y, 16) ||
        !aligned(mod_row, 4))
        return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        mf_status st = check_rows(mod_row, T, n_rows, s);
        if (st != MF_OK) return st;
    }
    mf::BlockOutArgs a;
    a.o = static_cast<const uint16_t*>(o);
    a.ld_o = ld_o;
    a.w = static_cast<const uint16_t*>(w_o);
    a.x = static_cast<const uint16_t*>(x);
    a.gate = static_cast<const uint16_t*>(gate);
    a.mod_row = mod_row;
    a.n_rows = n_rows;
    a.y = static_cast<uint16_t*>(y);
    a.T = T; a.C = C;
    return finish(mf::launch_block_out(a, s), s);
}

mf_status mf_cfg_euler_step(void* stream, const void* v, int64_t ld_v, const int32_t* rows, const float* z,
                            float* z_out, void* x_next, int64_t ld_x, int64_t n_tokens, int32_t Cl,
                            float guidance, float t, float t_next) {
    if (n_tokens < 0 || n_tokens > INT32_MAX || Cl <= 0 || Cl % 8 || Cl > 4096) return MF_ERR_SHAPE;
    if (ld_v < Cl || (x_next != nullptr && ld_x < Cl)) return MF_ERR_SHAPE;
    if (ld_v > kMaxStride || ld_x > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (!std::isfinite(guidance) || !std::isfinite(t) || !std::isfinite(t_next)) return MF_ERR_SHAPE;
    if (n_tokens == 0) return MF_OK;
    if (!v || !rows || !z || !z_out) return MF_ERR_NULL;
    if (ld_v % 8 || (x_next != nullptr && ld_x % 8)) return MF_ERR_ALIGN;
    if (!aligned(v, 16) || !aligned(rows, 8) || !aligned(z, 16) || !aligned(z_out, 16) ||
        (x_next != nullptr && !aligned(x_next, 16)))
        return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> hr;
        if (!fetch(rows, size_t(n_tokens) * 2, hr, s)) return MF_ERR_HIP;
        for (int32_t r : hr)
            if (r < 0) return MF_ERR_TABLE;
    }
    mf::CfgEulerArgs a;
    a.v = static_cast<const uint16_t*>(v);
    a.ld_v = ld_v;
    a.rows = rows;
    a.z = z;
    a.z_out = z_out;
    a.x_next = static_cast<uint16_t*>(x_next);
    a.ld_x = ld_x;
    a.N = n_tokens;
    a.Cl = Cl;
    a.w = guidance; a.t = t; a.t_next = t_next;
    return finish(mf::launch_cfg_euler(a, s), s);
}

mf_status mf_qk_norm_rope(void* stream, const void* q_in, int64_t ld_q, const void* k_in, int64_t ld_k,
                          void* q_out, int64_t ld_qo, void* k_out, int64_t ld_ko, const void* wq, const void* wk,
                          const int32_t* pos, int64_t T, int32_t Hq, int32_t Hkv, int32_t D, float rope_base,
                          float eps) {
    if (T < 0 || T > INT32_MAX || Hq <= 0 || Hkv <= 0) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (int64_t(Hq) * D > 8192 || int64_t(Hkv) * D > 8192) return MF_ERR_UNSUPPORTED;
    if (ld_q < int64_t(Hq) * D || ld_qo < int64_t(Hq) * D || ld_k < int64_t(Hkv) * D || ld_ko < int64_t(Hkv) * D)
        return MF_ERR_SHAPE;
    if (ld_q > kMaxStride || ld_qo > kMaxStride || ld_k > kMaxStride || ld_ko > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (!(rope_base > 0.f) || !std::isfinite(rope_base) || !(eps > 0.f)) return MF_ERR_SHAPE;
    if (T == 0) return MF_OK;
    if (!q_in || !k_in || !q_out || !k_out || !wq || !wk || !pos) return MF_ERR_NULL;
    if (ld_q % 8 || ld_k % 8 || ld_qo % 8 || ld_ko % 8) return MF_ERR_ALIGN;
    if (!aligned(q_in, 16) || !aligned(k_in, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
        !aligned(wq, 16) || !aligned(wk, 16) || !aligned(pos, 4))
        return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> hp;
        if (!fetch(pos, size_t(T), hp, s)) return MF_ERR_HIP;
        for (int32_t v : hp)
            if (v < 0) return MF_ERR_TABLE;
    }
    mf::QkNormRopeArgs a;
    a.q_in = static_cast<const uint16_t*>(q_in);
    a.k_in = static_cast<const uint16_t*>(k_in);
    a.q_out = static_cast<uint16_t*>(q_out);
    a.k_out = static_cast<uint16_t*>(k_out);
    a.ld_q = ld_q; a.ld_k = ld_k; a.ld_qo = ld_qo; a.ld_ko = ld_ko;
    a.wq = static_cast<const uint16_t*>(wq);
    a.wk = static_cast<const uint16_t*>(wk);
    a.pos = pos;
    a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
    a.rope_base = rope_base; a.eps = eps;
    return finish(mf::launch_qk_norm_rope(a, s), s);
}

size_t mf_varlen_attn_causal_workspace_bytes(int32_t n_seq, int64_t T) {
    if (!query_ok(T, 1, 1) || n_seq < 0 || n_seq > (1 << 24)) return 0;
    return mf::causal_attn_workspace_bytes(n_seq, T);
}

mf_status mf_varlen_attn_causal_fwd(void* stream, const void* q, int64_t ld_q, const void* k, const void* v,
                                    int64_t ld_kv, void* o, int64_t ld_o, float* lse, const int32_t* cu_seqlens,
                                    int32_t n_seq, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                    float softmax_scale, void* workspace, size_t workspace_bytes) {
    if (T < 0 || T > INT32_MAX || n_seq < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return MF_ERR_SHAPE;
    if (D != 64 && D != 128) return MF_ERR_UNSUPPORTED;
    if (ld_q < int64_t(Hq) * D || ld_o < int64_t(Hq) * D || ld_kv < int64_t(Hkv) * D) return MF_ERR_SHAPE;
    if (ld_q > kMaxStride || ld_o > kMaxStride || ld_kv > kMaxStride) return MF_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MF_ERR_SHAPE;
    if (T * ld_q * 2 >= (int64_t(1) << 32) || T * ld_kv * 2 >= (int64_t(1) << 32)) return MF_ERR_UNSUPPORTED;
    if (T == 0 || n_seq == 0) return MF_OK;
    if (!q || !k || !v || !o || !cu_seqlens) return MF_ERR_NULL;
    if (ld_q % 8 || ld_kv % 8 || ld_o % 8) return MF_ERR_ALIGN;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(cu_seqlens, 4) ||
        (lse && !aligned(lse, 4)))
        return MF_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < mf::causal_attn_workspace_bytes(n_seq, T)) return MF_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return MF_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
        std::vector<int32_t> hc;
        if (!fetch(cu_seqlens, size_t(n_seq) + 1, hc, s)) return MF_ERR_HIP;
        if (hc[0] != 0 || hc[n_seq] != T) return MF_ERR_TABLE;
        for (int32_t i = 0; i < n_seq; ++i)
            if (hc[i + 1] < hc[i]) return MF_ERR_TABLE;
    }
    mf::CausalAttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse; a.cu_seqlens = cu_seqlens; a.n_seq = n_seq;
    a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.D = D;
    a.ld_q = ld_q; a.ld_kv = ld_kv; a.ld_o = ld_o;
    a.softmax_scale = softmax_scale;
    a.workspace = workspace;
    return finish(mf::launch_varlen_attn_causal(a, s), s);
}

}  // extern "C"
