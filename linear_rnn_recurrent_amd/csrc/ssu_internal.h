// Internal interface between the C-ABI layer (ssu_api.cpp) and the kernel
// launchers (*.hip). Plain structs of device pointers and sizes; the host code
// has validated every field before a launcher sees it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssu.h"

namespace ssu {

struct DecodeParams {
    const void *x;
    const float *A;
    const void *B;
    const void *C;
    const float *dt;
    const float *dt_bias;
    const float *D;
    const void *z;
    void *state;
    void *out;
    const int32_t *idx;
    int64_t row_stride;  // elements
    int32_t batch, nheads, dim, dstate, ngroups;
    int32_t state_dtype, io_dtype, bc_dtype;
    int32_t dt_softplus;
};

struct PrefillParams {
    DecodeParams d;  // x/z/out/dt/B/C carry the extra seq_len axis
    int32_t seq_len;
    const int32_t *ctx;
    float *st_dA, *st_u, *st_B, *st_dt;  // all set or all null
    int32_t cu_count;                    // compute units of the device (workgroup ordering)
    int32_t waves_per_wg;                // 0: choose from the grid size; 4 or 8: forced
};

struct ReplayParams {
    void *state;
    const float *dA, *u, *B, *dt;
    const ssu_replay_layer *layers;  // device array; when set, the five pointers above are unused
    int32_t num_layers;
    const int32_t *accepted;
    const int32_t *idx;
    const int32_t *node_ids;  // null: token t is stash position t
    int64_t row_stride;
    int32_t active_batch, seq_len, nheads, dim, dstate, ngroups;
    int32_t state_dtype;
    int32_t max_accept_len;   // row length of node_ids
};

struct TreeParams {
    DecodeParams d;  // x/z/out/dt/B/C carry the node axis; the state is only read
    int32_t num_nodes;
    const int32_t *parents, *depths;
    float *st_dA, *st_u, *st_B, *st_dt;  // all set or all null
    float *gram;  // workspace: [batch][ngroups][M][M] fp32, B_j . C_m for j <= m
};

// One byte range to copy (src != null) or zero (src == null).
struct Segment {
    void *dst;
    const void *src;
    uint64_t bytes;
};

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_f16(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams &p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_f16(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams &p, hipStream_t stream);
hipError_t launch_replay(const ReplayParams &p, hipStream_t stream);
hipError_t launch_tree(const TreeParams &p, hipStream_t stream);
// Device address of the library's SSU_TREE_SCRATCH_BYTES tree scratch on the
// current device (looked up once per device).
hipError_t tree_scratch(void **ptr);
// Zeroes row `slot` (or all rows, slot -1) of both states of every layer.
hipError_t launch_clear_layers(const ssu_state_layer *layers, int num_layers, int rows, int slot,
                               int64_t rec_row_bytes, int64_t conv_row_bytes, hipStream_t stream);
hipError_t launch_tree_f32(const TreeParams &p, hipStream_t stream);
hipError_t launch_tree_f16(const TreeParams &p, hipStream_t stream);
hipError_t launch_tree_bf16(const TreeParams &p, hipStream_t stream);
struct GdnParams {
    const void *hs, *w_ba, *qkv, *conv_w, *conv_b;
    void *conv_state;
    const float *A_log;
    const void *dt_bias;
    float scale;
    float *ssm;
    const int32_t *idx;
    void *out;
    void *workspace;  // gdn_workspace_floats() fp32, 16-byte aligned
    int64_t ssm_row_stride, cs_slot, cs_chan, cs_tap;
    int32_t batch, hidden, hq, hv, dhead, width, use_l2;
};
int64_t gdn_workspace_floats(int64_t batch, int64_t hidden, int64_t hq, int64_t hv, int64_t d);
hipError_t launch_gdn(const GdnParams &p, hipStream_t stream);

// One set of row moves: for b < rows, dst row (dst_idx ? dst_idx[b] : b) gets
// src row (src_idx ? src_idx[b] : b); a negative destination index skips the
// row, a negative source index (or src == null) writes zeros; with skip_same,
// rows where skip_same[b] == b are not touched.
struct RowMove {
    void *dst;
    const void *src;
    const int32_t *dst_idx, *src_idx, *skip_same;
    int64_t dst_stride, src_stride;
    int32_t rows;
};
// Up to two row-move sets of row_bytes-byte rows in one launch.
hipError_t launch_row_moves(const RowMove *moves, int n, int64_t row_bytes, hipStream_t stream);
// Copies/zeroes up to any number of segments; one launch per 32 segments.
hipError_t launch_segments(const Segment *segs, int n, hipStream_t stream);

}  // namespace ssu
