// extern "C" entry points of libqkvattn.so: argument checks on the host, then launches.
// The declarations, argument meanings and layouts are in include/qkv_attn.h.
#include "launch.h"

using namespace qkv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int body_len(int n) { return n >= 64 ? 64 * ((n - 64) / 64) : 0; }

// Validates the descriptor and builds the by-value kernel argument.
int make_arg(const qkv_cache* c, CacheArg* a) {
    if (!c) return QKV_EINVAL;
    if (c->batch < 1 || c->heads < 1 || c->n_loops < 1) return QKV_EINVAL;
    if (c->head_dim != 64 && c->head_dim != 128) return QKV_EUNSUPPORTED;
    if (c->n_loops > QKV_MAX_LOOPS) return QKV_EUNSUPPORTED;
    if (c->cap_ctx < 64 || (c->cap_ctx % 64) != 0) return QKV_EINVAL;
    if (c->n_ctx < 0 || c->n_ctx > c->cap_ctx) return QKV_ECAPACITY;
    a->B = c->batch;
    a->H = c->heads;
    a->cap_ctx = c->cap_ctx;
    a->n_ctx = c->n_ctx;
    a->n_body = body_len(c->n_ctx);
    a->nplanes = c->n_loops;
    const int rb = c->residual_bits == 0 ? 4 : c->residual_bits;
    if (rb != 4 && rb != 2) return QKV_EUNSUPPORTED;
    if (c->full_state != 0 && c->full_state != 1) return QKV_EINVAL;
    if (c->full_state && rb != 4) return QKV_EUNSUPPORTED;  // the full-state codec is 4-bit
    a->rbits = rb;
    a->full = c->full_state;
    if (c->stored_loops && !aligned16(c->stored_loops)) return QKV_EINVAL;
    a->smask = c->stored_loops;
    a->eflags = c->error_flags;
    for (int p = 0; p < QKV_MAX_LOOPS; ++p) {
        PlaneArg& P = a->p[p];
        P = PlaneArg{};
        a->tail_k[p] = nullptr;
        a->tail_v[p] = nullptr;
        if (p >= c->n_loops) continue;
        const qkv_plane& s = c->plane[p];
        if (!s.data || !aligned16(s.data) || s.n_blocks < 1) return QKV_EINVAL;
        if (p == 0 && !s.dense) return QKV_EINVAL;  // the base stores every position
        if (s.dense) {
            if ((long)s.n_blocks * 64 < body_len(c->cap_ctx)) return QKV_ECAPACITY;
        } else {
            if (!s.rowmap || !s.rowpos || !s.rowstart) return QKV_EINVAL;
        }
        if (!c->tail_k[p] || !c->tail_v[p] || !aligned16(c->tail_k[p]) || !aligned16(c->tail_v[p]))
            return QKV_EINVAL;
        P.data = static_cast<const uint8_t*>(s.data);
        P.rowmap = s.rowmap;
        P.rowpos = s.rowpos;
        P.rowstart = s.rowstart;
        P.n_blocks = s.n_blocks;
        P.dense = s.dense ? 1 : 0;
        a->tail_k[p] = c->tail_k[p];
        a->tail_v[p] = c->tail_v[p];
    }
    return QKV_OK;
}

hipStream_t to_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Checks a tail-flush request of loop `loop` and builds its kernel argument (pos0 -1: none).
// The group must be the tail's 64 oldest rows, and must not hold the newest position.
int make_flush(const qkv_cache* c, int loop, const qkv_flush* f, FlushArg* out) {
    *out = FlushArg{-1};
    if (!f) return QKV_OK;
    const int nb = body_len(c->n_ctx);
    if (f->pos0 != nb || c->n_ctx < 64) return QKV_EINVAL;
    if ((long)f->pos0 + 64 > (long)c->n_ctx - 1) return QKV_EINVAL;
    if ((long)f->pos0 + 64 > c->cap_ctx) return QKV_ECAPACITY;
    const qkv_plane& P = c->plane[loop - 1];
    if (P.dense) {
        if (f->act_pos || f->n_act) return QKV_EINVAL;
        if ((long)f->pos0 + 64 > (long)P.n_blocks * 64) return QKV_ECAPACITY;
    } else {
        if (!f->act_pos || !f->n_act || f->ld_act < 1) return QKV_EINVAL;
    }
    out->pos0 = f->pos0;
    out->loop = loop;
    out->nch = c->full_state ? 0 : loop - 1;
    out->ld_act = f->ld_act;
    out->act_pos = P.dense ? nullptr : f->act_pos;
    out->n_act = P.dense ? nullptr : f->n_act;
    out->smask = P.dense ? nullptr : c->stored_loops;
    out->bit = 1u << (loop - 1);
    return QKV_OK;
}

}  // namespace

extern "C" {

const char* qkv_strerror(int status) {
    switch (status) {
        case QKV_OK: return "ok";
        case QKV_EINVAL: return "invalid argument";
        case QKV_EUNSUPPORTED: return "unsupported configuration";
        case QKV_ECAPACITY: return "capacity exceeded";
        case QKV_ELAUNCH: return "kernel launch failed";
        case QKV_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

size_t qkv_block_bytes(int head_dim, int bits) {
    if (bits == 4 && head_dim == 128) return Block<128, 4>::kBytes;
    if (bits == 4 && head_dim == 64) return Block<64, 4>::kBytes;
    if (bits == 2 && head_dim == 128) return Block<128, 2>::kBytes;
    if (bits == 2 && head_dim == 64) return Block<64, 2>::kBytes;
    return 0;
}

int qkv_body_len(int n_ctx) { return body_len(n_ctx); }

size_t qkv_workspace_bytes(int batch, int heads, int head_dim, int max_ctx, int max_k) {
    if (batch < 1 || heads < 1 || (head_dim != 64 && head_dim != 128) || max_ctx < 0 || max_k < 0) return 0;
    size_t need = 256;
    const int nb_max = body_len(max_ctx);
    for (int nb = 0; nb <= nb_max; nb += 64) {
        const size_t d = dense_ws_bytes(batch, heads, head_dim, nb);
        need = d > need ? d : need;
    }
    const size_t s = sparse_ws_bytes(batch, heads, head_dim, max_k);
    need = s > need ? s : need;
    const size_t t = select_ws_bytes(batch, heads, max_ctx);
    need = t > need ? t : need;
    return (need + 255) & ~(size_t)255;
}

int kv_encode_loop(const qkv_cache* cache, int loop, int pos0, int n_pos, const int32_t* act_pos,
                   const int32_t* n_act, int ld_act, const uint16_t* k_src, const uint16_t* v_src, int ld_src,
                   void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 1 || loop > cache->n_loops) return QKV_EINVAL;
    if (pos0 < 0 || (pos0 % 64) != 0 || n_pos <= 0 || (n_pos % 64) != 0) return QKV_EINVAL;
    if ((long)pos0 + n_pos > cache->cap_ctx) return QKV_ECAPACITY;
    const qkv_plane& P = cache->plane[loop - 1];
    if (P.dense) {
        if (act_pos || n_act) return QKV_EINVAL;
        if ((long)(pos0 + n_pos) > (long)P.n_blocks * 64) return QKV_ECAPACITY;
    } else {
        if (!act_pos || !n_act || ld_act < 1) return QKV_EINVAL;
    }
    if ((k_src == nullptr) != (v_src == nullptr)) return QKV_EINVAL;
    if (k_src) {
        if (!aligned16(k_src) || !aligned16(v_src)) return QKV_EINVAL;
        if (ld_src < n_pos) return QKV_EINVAL;
    } else {
        // flush from the BF16 tail: the positions must be tail positions of the current context
        if (pos0 < body_len(cache->n_ctx) || (long)pos0 + n_pos > cache->n_ctx) return QKV_EINVAL;
        if (cache->n_ctx - pos0 > QKV_TAIL_SLOTS) return QKV_EINVAL;
        ld_src = 0;
    }
    return launch_encode(a, cache->head_dim, loop, pos0, n_pos, act_pos, n_act, ld_act, k_src, v_src, ld_src,
                         to_stream(stream));
}

int kv_append_tail(const qkv_cache* cache, int loop, int pos0, int n_rows, const uint16_t* k, const uint16_t* v,
                   void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 0 || loop > cache->n_loops) return QKV_EINVAL;
    if (n_rows < 1 || n_rows > QKV_TAIL_SLOTS || pos0 < 0) return QKV_EINVAL;
    if ((long)pos0 + n_rows > cache->cap_ctx) return QKV_ECAPACITY;
    if (!k || !v || !aligned16(k) || !aligned16(v)) return QKV_EINVAL;
    if (loop == 0) return launch_append_all(a, cache->head_dim, pos0, n_rows, k, v, to_stream(stream));
    return launch_append(cache->batch, cache->heads, cache->head_dim, pos0, n_rows, k, v, cache->tail_k[loop - 1],
                         cache->tail_v[loop - 1], to_stream(stream));
}

int attn_decode_dense(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, float sm_scale, uint16_t* o, float* o_f32, float* scores,
                      int ld_scores, float* lse, const qkv_flush* flush, void* ws, size_t ws_bytes, void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 1 || loop > cache->n_loops) return QKV_EINVAL;
    if (cache->n_ctx < 1) return QKV_EINVAL;
    if (!q || !o_f32 || !lse || (scores && ld_scores < cache->n_ctx)) return QKV_EINVAL;
    if (!aligned16(q) || !aligned16(o_f32) || (o && !aligned16(o))) return QKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr) || (k_new && (!aligned16(k_new) || !aligned16(v_new))))
        return QKV_EINVAL;
    FlushArg fl;
    st = make_flush(cache, loop, flush, &fl);
    if (st) return st;
    const size_t need = dense_ws_bytes(cache->batch, cache->heads, cache->head_dim, a.n_body);
    if (!ws || ws_bytes < need) return QKV_EWORKSPACE;
    return launch_dense(a, cache->head_dim, loop, q, NewRow{k_new, v_new}, sm_scale, o, o_f32, scores, ld_scores,
                        lse, ws, to_stream(stream), fl);
}

int attn_decode_dense_noalloc(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                              const uint16_t* v_new, float sm_scale, uint16_t* o, float* o_f32, float* scores,
                              int ld_scores, float* lse, void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 1 || loop > cache->n_loops) return QKV_EINVAL;
    if (cache->n_ctx < 1) return QKV_EINVAL;
    if (!q || !o_f32 || !lse || (scores && ld_scores < cache->n_ctx)) return QKV_EINVAL;
    if (!aligned16(q) || !aligned16(o_f32) || (o && !aligned16(o))) return QKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr) || (k_new && (!aligned16(k_new) || !aligned16(v_new))))
        return QKV_EINVAL;
    return launch_dense_noalloc(a, cache->head_dim, loop, q, NewRow{k_new, v_new}, sm_scale, o, o_f32, scores,
                                ld_scores, lse, to_stream(stream));
}

int select_columns(const float* scores, int ld_scores, const float* lse, int batch, int heads, int n, int k,
                   int32_t* idx, float* p_sel, float* mass, void* ws, size_t ws_bytes, void* stream) {
    if (!scores || !lse || !mass || batch < 1 || heads < 1 || n < 1 || ld_scores < n) return QKV_EINVAL;
    if (k < 0 || k > n) return QKV_EINVAL;
    if (k > 0 && (!idx || !p_sel)) return QKV_EINVAL;
    if (ws_bytes < select_ws_bytes(batch, heads, n)) return QKV_EWORKSPACE;
    return launch_select(scores, ld_scores, lse, batch, heads, n, k, idx, p_sel, mass, ws, to_stream(stream));
}

int select_tokens(const uint16_t* h_cur, const uint16_t* h_prev, int ld_tok, int batch, int n, int dm,
                  const int32_t* act_prev, const int32_t* n_act_prev, int ld_act, int k, int split, float* score,
                  int32_t* act_out, int32_t* n_act_out, int32_t* n_before, void* ws, size_t ws_bytes, void* stream) {
    if (!h_cur || !h_prev || !score || !act_out || !n_act_out) return QKV_EINVAL;
    if (batch < 1 || n < 1 || dm < 8 || (dm % 8) != 0 || ld_tok < n) return QKV_EINVAL;
    if (!aligned16(h_cur) || !aligned16(h_prev)) return QKV_EINVAL;
    if (k < 1 || k > n) return QKV_EINVAL;
    if ((act_prev == nullptr) != (n_act_prev == nullptr)) return QKV_EINVAL;
    if (act_prev && (ld_act < 1 || ld_act > n)) return QKV_EINVAL;
    if (!ws || ws_bytes < token_ws_bytes(batch, k)) return QKV_EWORKSPACE;
    return launch_select_tokens(h_cur, h_prev, ld_tok, batch, n, dm, act_prev, n_act_prev, ld_act, k, split, score,
                                act_out, n_act_out, n_before, ws, to_stream(stream));
}

size_t qkv_token_workspace_bytes(int batch, int k) {
    if (batch < 1 || k < 1) return 0;
    return (token_ws_bytes(batch, k) + 255) & ~(size_t)255;
}

int attn_decode_sparse(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                       const uint16_t* v_new, float sm_scale, const int32_t* idx,
                       const float* p_sel, const float* mass, int k, const float* o_prev, const float* lse,
                       float* scores, int ld_scores, uint16_t* o, float* o_f32, const qkv_flush* flush, void* ws,
                       size_t ws_bytes, void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 2 || loop > cache->n_loops) return QKV_EINVAL;
    if (cache->n_ctx < 1 || k < 0 || k > cache->n_ctx) return QKV_EINVAL;
    if (!q || !o_prev || !lse || !o_f32 || (scores && ld_scores < cache->n_ctx)) return QKV_EINVAL;
    if (k > 0 && (!idx || !p_sel || !mass)) return QKV_EINVAL;
    if (!aligned16(q) || (o && !aligned16(o))) return QKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr) || (k_new && (!aligned16(k_new) || !aligned16(v_new))))
        return QKV_EINVAL;
    FlushArg fl;
    st = make_flush(cache, loop, flush, &fl);
    if (st) return st;
    const size_t need = sparse_ws_bytes(cache->batch, cache->heads, cache->head_dim, k);
    if (k > 0 && (!ws || ws_bytes < need)) return QKV_EWORKSPACE;
    return launch_sparse(a, cache->head_dim, loop, q, NewRow{k_new, v_new}, sm_scale, idx, p_sel, mass, k, o_prev,
                         lse, scores, ld_scores, o, o_f32, ws, to_stream(stream), fl);
}

int qkv_export_plane(const qkv_cache* cache, int loop, int b, int h, int n_slots, uint8_t* k_codes,
                     uint8_t* v_codes, float* k_scale, float* k_zero, float* v_scale, float* v_zero, void* stream) {
    CacheArg a;
    int st = make_arg(cache, &a);
    if (st) return st;
    if (loop < 1 || loop > cache->n_loops || b < 0 || b >= cache->batch || h < 0 || h >= cache->heads)
        return QKV_EINVAL;
    if (n_slots < 1 || (long)n_slots > (long)cache->plane[loop - 1].n_blocks * 64) return QKV_EINVAL;
    if (!k_codes || !v_codes || !k_scale || !k_zero || !v_scale || !v_zero) return QKV_EINVAL;
    return launch_export_plane(a, cache->head_dim, loop, b, h, n_slots, k_codes, v_codes, k_scale, k_zero, v_scale,
                               v_zero, to_stream(stream));
}

int kv_gather_rows(const uint16_t* src, int batch, int heads, int ld_src, int head_dim, const int32_t* idx, int n_idx,
                   int idx_per_head, int transpose, uint16_t* dst, void* stream) {
    if (!src || !idx || !dst || batch < 1 || heads < 1 || ld_src < 1 || n_idx < 1) return QKV_EINVAL;
    if (head_dim != 64 && head_dim != 128) return QKV_EUNSUPPORTED;
    if ((idx_per_head != 0 && idx_per_head != 1) || (transpose != 0 && transpose != 1)) return QKV_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return QKV_EINVAL;
    return launch_gather_rows(src, batch, heads, ld_src, head_dim, idx, n_idx, idx_per_head, transpose, dst,
                              to_stream(stream));
}

int attn_prefill_sparse(int batch, int heads, int head_dim, const uint16_t* q, const uint16_t* q_prev,
                        const int32_t* q_pos, int n_q, const float* lse_prev, const float* o_prev, const uint16_t* k,
                        const uint16_t* k_prev, const uint16_t* v_t, const uint16_t* v_prev_t, const int32_t* c_pos,
                        int n_c, float sm_scale, float* o_f32, uint16_t* o, float* mass, void* stream) {
    if (batch < 1 || heads < 1 || n_q < 1 || n_c < 0) return QKV_EINVAL;
    if (head_dim != 64 && head_dim != 128) return QKV_EUNSUPPORTED;
    if (!q || !q_prev || !q_pos || !lse_prev || !o_prev || !o_f32) return QKV_EINVAL;
    if (n_c > 0 && (!k || !k_prev || !v_t || !v_prev_t || !c_pos)) return QKV_EINVAL;
    if (!aligned16(q) || !aligned16(q_prev) || !aligned16(o_prev) || !aligned16(o_f32) || (o && !aligned16(o)))
        return QKV_EINVAL;
    if (n_c > 0 && (!aligned16(k) || !aligned16(k_prev) || !aligned16(v_t) || !aligned16(v_prev_t)))
        return QKV_EINVAL;
    return launch_prefill_sparse(batch, heads, head_dim, q, q_prev, q_pos, n_q, lse_prev, o_prev, k, k_prev, v_t,
                                 v_prev_t, c_pos, n_c, sm_scale, o_f32, o, mass, to_stream(stream));
}

int qkv_stream_read(const void* src, size_t n_bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || n_bytes == 0 || (n_bytes % 16) != 0 || !aligned16(src) || !aligned16(sink))
        return QKV_EINVAL;
    return launch_stream_read(src, n_bytes, sink, to_stream(stream));
}

}  // extern "C"
