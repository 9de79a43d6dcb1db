// Internal launchers shared by the kernel translation units and the C ABI.
#pragma once

#include "common.h"

namespace qkv {

int launch_encode(const CacheArg& ca, int D, int loop, int pos0, int n_pos, const int32_t* act_pos,
                  const int32_t* n_act, int ld_act, const uint16_t* ksrc, const uint16_t* vsrc, int ld_src,
                  hipStream_t st);
int launch_append(int B, int H, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v, uint16_t* tk,
                  uint16_t* tv, hipStream_t st);
int launch_append_all(const CacheArg& ca, int D, int pos0, int n_rows, const uint16_t* k, const uint16_t* v,
                      hipStream_t st);

// The newest position's row of one loop (bf16 [B][H][D] each), or both NULL.
struct NewRow {
    const uint16_t* k;
    const uint16_t* v;
};

// The 64-row tail flush of one loop, encoded by extra workgroups of that loop's attention
// kernel in the step before the body boundary moves: no reader of that step touches the
// group (its positions are still tail positions), so the roles are independent.
struct FlushArg {
    int32_t pos0;            // first position of the group (the body length); -1: no flush
    int32_t loop;            // the loop encoded, in the kernel argument's plane numbering
    int32_t nch;             // planes of the chain (loop - 1; 0 for the full-state codec)
    int32_t ld_act;
    const int32_t* act_pos;  // sparse plane: the group's active positions, ascending; else null
    const int32_t* n_act;
    uint32_t* smask;         // stored-loops words kept for sparse planes, or null
    uint32_t bit;
};
// extra workgroups per (head, sequence) for a flush: keys, values, and the maps of a sparse plane
inline int flush_groups(const FlushArg& f, bool sparse_plane) { return f.pos0 < 0 ? 0 : (sparse_plane ? 3 : 2); }

// split-KV plan of the dense reader: blocks per split and number of body splits
struct DensePlan {
    int spb;
    int nsplit;
};
DensePlan dense_plan(int B, int H, int n_body);
// Full-state codec: the cache argument seen from the last dense plane at or before `loop`
// (plane 0 of the result); *loop_out = the loop's index in it.
CacheArg full_state_view(const CacheArg& ca, int loop, int* loop_out);
size_t dense_ws_bytes(int B, int H, int D, int n_body);
int launch_dense(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o, float* o32,
                 float* scores, int ld, float* lse, void* ws, hipStream_t st, FlushArg fl = FlushArg{-1});

int launch_dense_noalloc(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o,
                         float* o32, float* scores, int ld, float* lse, hipStream_t st);

size_t select_ws_bytes(int B, int H, int n);
int launch_select(const float* scores, int ld, const float* lse, int B, int H, int n, int k, int32_t* idx,
                  float* p_sel, float* mass, void* ws, hipStream_t st);

int launch_export_plane(const CacheArg& ca, int D, int loop, int b, int h, int n_slots, uint8_t* kc, uint8_t* vc,
                        float* ks, float* kz, float* vs, float* vz, hipStream_t st);

size_t token_ws_bytes(int B, int k);
int launch_select_tokens(const uint16_t* hc, const uint16_t* hp, int ld_tok, int B, int n, int dm,
                         const int32_t* act, const int32_t* n_act, int ld_act, int k, int split, float* score,
                         int32_t* act_out, int32_t* n_out, int32_t* n_before, void* ws, hipStream_t st);

int launch_gather_rows(const uint16_t* src, int B, int H, int ld_src, int D, const int32_t* idx, int n, int per_head,
                       int transpose, uint16_t* dst, hipStream_t st);
int launch_prefill_sparse(int B, int H, int D, const uint16_t* q1, const uint16_t* q0, const int32_t* qpos, int n_q,
                          const float* lse0, const float* o0, const uint16_t* k1, const uint16_t* k0,
                          const uint16_t* v1t, const uint16_t* v0t, const int32_t* cpos, int n_c, float sm,
                          float* o32, uint16_t* o16, float* mass, hipStream_t st);

int launch_stream_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t st);
size_t sparse_ws_bytes(int B, int H, int D, int k);
int launch_sparse(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, const int32_t* idx,
                  const float* p_sel, const float* mass, int k, const float* o_prev, const float* lse,
                  float* scores, int ld, uint16_t* o, float* o32, void* ws, hipStream_t st, FlushArg fl = FlushArg{-1});

}  // namespace qkv
