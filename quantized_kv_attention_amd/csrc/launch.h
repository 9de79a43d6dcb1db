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

// split-KV plan of the dense reader: blocks per split and number of body splits
struct DensePlan {
    int spb;
    int nsplit;
};
DensePlan dense_plan(int B, int H, int n_body);
size_t dense_ws_bytes(int B, int H, int D, int n_body);
int launch_dense(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, uint16_t* o, float* o32,
                 float* scores, int ld, float* lse, void* ws, hipStream_t st);

size_t select_ws_bytes(int B, int H, int n);
int launch_select(const float* scores, int ld, const float* lse, int B, int H, int n, int k, int32_t* idx,
                  float* p_sel, float* mass, void* ws, hipStream_t st);

int launch_stream_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t st);
size_t sparse_ws_bytes(int B, int H, int D, int k);
int launch_sparse(const CacheArg& ca, int D, int loop, const uint16_t* q, NewRow nr, float sm, const int32_t* idx,
                  const float* p_sel, const float* mass, int k, const float* o_prev, const float* lse,
                  float* scores, int ld, uint16_t* o, float* o32, void* ws, hipStream_t st);

}  // namespace qkv
