// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libmf.so.  Not part of the public interface (include/mf.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace mf {

// Compute units of the current device (0 when none is visible).
int device_cu_count();

// ---------------------------------------------------------------------------
// Launchers (one per kernel family).  Arguments are already validated by the
// C-ABI layer; each returns the hipError_t of its launches.
// ---------------------------------------------------------------------------

struct ModRopeArgs {
    const uint16_t* q_in;
    const uint16_t* k_in;
    uint16_t* q_out;
    uint16_t* k_out;
    int64_t T;
    int32_t H, D;
    int64_t ld_in, ld_out;
    const uint16_t* shift;   // nullptr: RoPE only
    const uint16_t* scale;
    const int32_t* mod_row;
    int32_t n_rows;          // rows of shift/scale; a row outside [0, n_rows) reads zeros
    const int32_t* pos;
    int32_t rope_f, rope_r, rope_c;
    float rope_base, eps;
    // Rotation frequency of every pair of a head (index = dim / 2) in turns
    // per position, filled by the launcher in double precision:
    // base^(-2j / D_axis) / (2 pi).
    double theta_turns[64];
};
hipError_t launch_modulate_rope(const ModRopeArgs& a, hipStream_t stream);

struct ModRopeBwdArgs {
    const uint16_t* q_in;     // forward inputs
    const uint16_t* k_in;
    const uint16_t* dq_out;   // gradients of the forward outputs
    const uint16_t* dk_out;
    uint16_t* dq_in;          // gradients of the forward inputs (written)
    uint16_t* dk_in;
    int64_t T;
    int32_t H, D;
    int64_t ld_in, ld_gout, ld_gin;
    const uint16_t* scale;    // nullptr: RoPE only
    const int32_t* mod_row;
    int32_t n_rows;
    float* dshift;            // fp32 [n_rows][H*D] (written)
    float* dscale;
    const int32_t* pos;
    int32_t rope_f, rope_r, rope_c;
    float rope_base, eps;
    void* workspace;          // row-sum slots (modulated only)
    double theta_turns[64];   // filled by the launcher, as for the forward
};
hipError_t launch_modulate_rope_bwd(const ModRopeBwdArgs& a, hipStream_t stream);

struct GatedResBwdArgs {
    const uint16_t* x;
    const uint16_t* o;
    const uint16_t* gate;
    const int32_t* mod_row;
    int32_t n_rows;
    const uint16_t* dy;       // nullptr: zero
    const uint16_t* scale2;   // nullptr with dz: no fused adaLN
    const uint16_t* dz;
    uint16_t* dx;
    uint16_t* dout;           // gradient of the attention output o
    float* dgate;             // fp32 [n_rows][C] (written)
    float* dshift2;
    float* dscale2;
    int64_t T;
    int32_t C;
    float eps;
    void* workspace;          // row-sum slots
};
hipError_t launch_gated_residual_bwd(const GatedResBwdArgs& a, hipStream_t stream);
// Workspace of the two elementwise backward kernels: tagged row-sum slots of
// n_arrays x C floats per run of tokens.
size_t elementwise_bwd_workspace_bytes(int64_t T, int32_t C, int32_t n_arrays);

struct GatedResArgs {
    const uint16_t* x;
    const uint16_t* o;
    uint16_t* y;
    const uint16_t* gate;
    const int32_t* mod_row;
    int32_t n_rows;          // rows of gate/shift2/scale2; a row outside [0, n_rows) reads zeros
    const uint16_t* shift2;  // nullptr: no fused adaLN
    const uint16_t* scale2;
    uint16_t* z;
    int64_t T;
    int32_t C;
    float eps;
};
hipError_t launch_gated_residual(const GatedResArgs& a, hipStream_t stream);

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* cu_seqlens;
    int32_t n_seq, max_seqlen;
    int64_t T;
    int32_t H, D;
    int64_t ld_qkv, ld_o;
    float softmax_scale;
    void* workspace;
    size_t workspace_bytes;
};
size_t attn_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D);
hipError_t launch_varlen_attn_fwd(const AttnArgs& a, hipStream_t stream);
// Allocation-free forward: the workspace is the library's per-GPU scratch
// array of kAttnNoAllocScratchBytes.
constexpr size_t kAttnNoAllocScratchBytes = size_t(80) << 20;
hipError_t launch_varlen_attn_fwd_noalloc(const AttnArgs& a, hipStream_t stream);
// Persistent grid of the attention forward: g > 0 overrides one workgroup
// per CU (tests move the stream-K cut points with it); 0 restores it.
void set_attn_fwd_grid(int g);

struct AttnBwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const int32_t* cu_seqlens;
    int32_t n_seq, max_seqlen;
    int64_t T;
    int32_t H, D;
    int64_t ld_qkv, ld_o, ld_d;
    float softmax_scale;
    void* workspace;
    size_t workspace_bytes;
};
size_t attn_bwd_workspace_bytes(int32_t n_seq, int64_t T, int32_t H, int32_t D);
hipError_t launch_varlen_attn_bwd(const AttnBwdArgs& a, hipStream_t stream);

// Block projections around the attention: the QKV projection of the
// adaLN-modulated residual stream with RoPE on q and k, and the out
// projection with the gated residual.
struct BlockQkvArgs {
    const uint16_t* x;        // [T][C], token stride ld_x
    int64_t ld_x;
    const uint16_t* w;        // [3C][C]
    uint16_t* qkv;            // [T][3C], token stride ld_qkv
    int64_t ld_qkv;
    const uint16_t* shift;    // nullptr: no modulation
    const uint16_t* scale;
    const int32_t* mod_row;
    int32_t n_rows;           // rows of shift/scale; a row outside [0, n_rows) reads zeros
    const int32_t* pos;
    int64_t T;
    int32_t H, D;
    int32_t rope_f, rope_r, rope_c;
    float rope_base, eps;
    void* workspace;          // modulated rows bf16 [T][C], rotation table fp32 [T][D/2][2], partial tiles
};
size_t block_qkv_workspace_bytes(int64_t T, int32_t C, int32_t D);
hipError_t launch_block_qkv(const BlockQkvArgs& a, hipStream_t stream);

struct BlockOutArgs {
    const uint16_t* o;        // [T][C], token stride ld_o
    int64_t ld_o;
    const uint16_t* w;        // [C][C]
    const uint16_t* x;        // [T][C] residual
    const uint16_t* gate;     // [n_rows][C]
    const int32_t* mod_row;
    int32_t n_rows;           // a row outside [0, n_rows) reads zeros
    uint16_t* y;              // [T][C]
    int64_t T;
    int32_t C;
};
hipError_t launch_block_out(const BlockOutArgs& a, hipStream_t stream);

// Packed classifier-free guidance + Euler step over the evolving latents.
struct CfgEulerArgs {
    const uint16_t* v;        // bf16 velocities of the packed batch, [T][Cl] with token stride ld_v
    int64_t ld_v;
    const int32_t* rows;      // [N][2] packed rows of the conditional and unconditional copy
    const float* z;           // fp32 state [N][Cl]
    float* z_out;             // fp32 [N][Cl] (may equal z)
    uint16_t* x_next;         // nullptr, or bf16 rows [T][Cl] with token stride ld_x
    int64_t ld_x;
    int64_t N;
    int32_t Cl;
    float w, t, t_next;
};
hipError_t launch_cfg_euler(const CfgEulerArgs& a, hipStream_t stream);

// Text-encoder variant: per-head RMS norm + 1D RoPE of q and k, and causal
// attention with grouped key/value heads over packed prompts.
struct QkNormRopeArgs {
    const uint16_t* q_in;     // [T][Hq][D], token stride ld_q
    const uint16_t* k_in;     // [T][Hkv][D], token stride ld_k
    uint16_t* q_out;          // token stride ld_qo
    uint16_t* k_out;          // token stride ld_ko
    int64_t ld_q, ld_k, ld_qo, ld_ko;
    const uint16_t* wq;       // [D]
    const uint16_t* wk;       // [D]
    const int32_t* pos;       // [T] index inside the prompt
    int64_t T;
    int32_t Hq, Hkv, D;
    float rope_base, eps;
    double theta_turns[64];   // filled by the launcher: base^(-2j/D) / (2 pi)
};
hipError_t launch_qk_norm_rope(const QkNormRopeArgs& a, hipStream_t stream);

struct CausalAttnArgs {
    const uint16_t* q;        // [T][Hq][D], token stride ld_q
    const uint16_t* k;        // [T][Hkv][D], token stride ld_kv
    const uint16_t* v;
    uint16_t* o;              // [T][Hq][D], token stride ld_o
    float* lse;               // nullable, [Hq][T]
    const int32_t* cu_seqlens;
    int32_t n_seq;
    int64_t T;
    int32_t Hq, Hkv, D;
    int64_t ld_q, ld_kv, ld_o;
    float softmax_scale;
    void* workspace;          // slab descriptors, causal_attn_workspace_bytes
};
size_t causal_attn_workspace_bytes(int32_t n_seq, int64_t T);
hipError_t launch_varlen_attn_causal(const CausalAttnArgs& a, hipStream_t stream);

}  // namespace mf
