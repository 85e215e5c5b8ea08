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
        const int64_t img = int64_t(e.n_frames) * int64_t(e.grid_h) * int64_t(e.grid_w);
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
    if (cu_seqlens == nullptr || pos == nullptr) return MF_ERR_NULL;
    int64_t T = 0;
    mf_status st = count_tokens(descs, n, &T);
    if (st != MF_OK) return st;
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
        // Frames in order, each frame's grid in row-major (raster) order.
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
