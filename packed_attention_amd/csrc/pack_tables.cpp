// Host-side integer pack tables: cumulative offsets, per-token (frame, row,
// col) positions, sample ids and adaLN rows.
//
// Packing with per-sample cumulative offsets under a token budget: picx.dev
// summary of Mage-Flow, Methodology > Native-Resolution MMDiT.  Per-sample
// 2D positions for the rotary embedding: gist.science "Resumo Tecnico:
// Mage-Flow", Metodologia > 2. NR-MMDiT.  Frame axis for edit source and
// target latents: picx.dev summary, same section, conditioning item.
//
// Plain C++ with no HIP dependency, so it also builds and runs under the
// host sanitizers.
#include <climits>
#include <cstdint>

#include "mf.h"

namespace {

mf_status count_tokens(const mf_sample_desc* d, int32_t n, int64_t* total) {
    if (n < 0) return MF_ERR_SHAPE;
    if (n > 0 && d == nullptr) return MF_ERR_NULL;
    int64_t T = 0;
    for (int32_t s = 0; s < n; ++s) {
        const mf_sample_desc& e = d[s];
        if (e.text_len < 0 || e.n_frames < 0 || e.grid_h < 0 || e.grid_w < 0 ||
            e.mod_row_text < 0 || e.mod_row_image < 0)
            return MF_ERR_SHAPE;
        // frames * rows * cols, checked after each product (each fits int64
        // because its factors are below 2^31)
        int64_t img = int64_t(e.n_frames) * int64_t(e.grid_h);
        if (img > INT32_MAX && e.grid_w > 0) return MF_ERR_SHAPE;
        img = e.grid_w == 0 ? 0 : img * int64_t(e.grid_w);
        if (img > INT32_MAX) return MF_ERR_SHAPE;
        T += int64_t(e.text_len) + img;
        if (T > INT32_MAX) return MF_ERR_SHAPE;
    }
    *total = T;
    return MF_OK;
}

}  // namespace

extern "C" mf_status mf_pack_count(const mf_sample_desc* descs, int32_t n, int64_t* total_tokens) {
    if (total_tokens == nullptr) return MF_ERR_NULL;
    return count_tokens(descs, n, total_tokens);
}

extern "C" mf_status mf_pack_tables(const mf_sample_desc* descs, int32_t n, int32_t* cu_seqlens,
                                    int32_t* pos, int32_t* seq_id, int32_t* mod_row) {
    if (cu_seqlens == nullptr) return MF_ERR_NULL;
    int64_t T = 0;
    mf_status st = count_tokens(descs, n, &T);
    if (st != MF_OK) return st;
    if (pos == nullptr && T > 0) return MF_ERR_NULL;
    int32_t t = 0;
    cu_seqlens[0] = 0;
    for (int32_t s = 0; s < n; ++s) {
        const mf_sample_desc& e = descs[s];
        for (int32_t j = 0; j < e.text_len; ++j, ++t) {
            pos[3 * t + 0] = 0;
            pos[3 * t + 1] = 0;
            pos[3 * t + 2] = 0;
            if (seq_id) seq_id[t] = s;
            if (mod_row) mod_row[t] = e.mod_row_text;
        }
        // Frames in order, each frame's grid in row-major (raster) order (an
        // empty grid has no tokens, whatever the frame count and other side).
        if (e.grid_h > 0 && e.grid_w > 0)
        for (int32_t f = 0; f < e.n_frames; ++f)
            for (int32_t r = 0; r < e.grid_h; ++r)
                for (int32_t c = 0; c < e.grid_w; ++c, ++t) {
                    pos[3 * t + 0] = f;
                    pos[3 * t + 1] = r;
                    pos[3 * t + 2] = c;
                    if (seq_id) seq_id[t] = s;
                    if (mod_row) mod_row[t] = e.mod_row_image;
                }
        cu_seqlens[s + 1] = t;
    }
    return MF_OK;
}

// ---------------------------------------------------------------------------
// Packed classifier-free guidance: the conditional and unconditional copies
// of a prompt run as two samples of one pack (picx.dev summary,
// Methodology > Native-Resolution MMDiT).  The latents that the sampler step
// moves are the last frame's (generation: the only frame; editing: the
// target frame, after the source frame), h*w tokens in raster order after
// the sample's text and earlier frames.
// ---------------------------------------------------------------------------
namespace {

mf_status cfg_count(const mf_sample_desc* d, int32_t n, const int32_t* cond, const int32_t* uncond,
                    int32_t P, int64_t* total) {
    int64_t T = 0;
    mf_status st = count_tokens(d, n, &T);
    if (st != MF_OK) return st;
    if (P < 0) return MF_ERR_SHAPE;
    if (P > 0 && (cond == nullptr || uncond == nullptr)) return MF_ERR_NULL;
    int64_t N = 0;
    for (int32_t p = 0; p < P; ++p) {
        const int32_t c = cond[p], u = uncond[p];
        if (c < 0 || c >= n || u < 0 || u >= n || c == u) return MF_ERR_SHAPE;
        if (d[c].n_frames < 1 || d[u].n_frames < 1) return MF_ERR_SHAPE;
        if (d[c].grid_h != d[u].grid_h || d[c].grid_w != d[u].grid_w) return MF_ERR_SHAPE;
        N += int64_t(d[c].grid_h) * d[c].grid_w;
    }
    *total = N;
    return MF_OK;
}

}  // namespace

extern "C" mf_status mf_cfg_pair_count(const mf_sample_desc* descs, int32_t n, const int32_t* cond,
                                       const int32_t* uncond, int32_t n_prompts, int64_t* n_tokens) {
    if (n_tokens == nullptr) return MF_ERR_NULL;
    return cfg_count(descs, n, cond, uncond, n_prompts, n_tokens);
}

extern "C" mf_status mf_cfg_pair_rows(const mf_sample_desc* descs, int32_t n, const int32_t* cond,
                                      const int32_t* uncond, int32_t n_prompts, int32_t* rows) {
    int64_t N = 0;
    mf_status st = cfg_count(descs, n, cond, uncond, n_prompts, &N);
    if (st != MF_OK) return st;
    if (N > 0 && rows == nullptr) return MF_ERR_NULL;
    // sample starts (cumulative offsets)
    int64_t k = 0;
    for (int32_t p = 0; p < n_prompts; ++p) {
        const int32_t c = cond[p], u = uncond[p];
        int64_t bc = 0, bu = 0, off = 0;
        for (int32_t s = 0; s < n; ++s) {
            if (s == c) bc = off;
            if (s == u) bu = off;
            off += int64_t(descs[s].text_len) + int64_t(descs[s].n_frames) * descs[s].grid_h * descs[s].grid_w;
        }
        const int64_t hw = int64_t(descs[c].grid_h) * descs[c].grid_w;
        bc += descs[c].text_len + int64_t(descs[c].n_frames - 1) * hw;
        bu += descs[u].text_len + int64_t(descs[u].n_frames - 1) * hw;
        for (int64_t j = 0; j < hw; ++j, ++k) {
            rows[2 * k] = int32_t(bc + j);
            rows[2 * k + 1] = int32_t(bu + j);
        }
    }
    return MF_OK;
}

// ---------------------------------------------------------------------------
// Packed prompts of the text encoder: cumulative offsets and every token's
// index inside its prompt (the rotary position of the causal encoder).
// ---------------------------------------------------------------------------
extern "C" mf_status mf_prompt_tables(const int32_t* lens, int32_t n, int32_t* cu_seqlens, int32_t* pos) {
    if (n < 0) return MF_ERR_SHAPE;
    if (cu_seqlens == nullptr || (n > 0 && lens == nullptr)) return MF_ERR_NULL;
    int64_t T = 0;
    for (int32_t s = 0; s < n; ++s) {
        if (lens[s] < 0) return MF_ERR_SHAPE;
        T += lens[s];
        if (T > INT32_MAX) return MF_ERR_SHAPE;
    }
    if (T > 0 && pos == nullptr) return MF_ERR_NULL;
    int32_t t = 0;
    cu_seqlens[0] = 0;
    for (int32_t s = 0; s < n; ++s) {
        for (int32_t j = 0; j < lens[s]; ++j) pos[t++] = j;
        cu_seqlens[s + 1] = t;
    }
    return MF_OK;
}
