// sa_api.cpp -- the C entry points declared in include/sa.h: admission,
// argument checks, then the launches on the caller's stream.  Nothing here
// allocates, copies or synchronises.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "sa.h"
#include "sa_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

sa_status check_ptrs(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (!p) return SA_ERR_NULL;
    for (const void* p : ptrs)
        if (!aligned16(p)) return SA_ERR_ALIGN;
    return SA_OK;
}

bool scale_ok(float x) { return isfinite(x) && x > 0.0f; }

sa::Shape to_shape(const sa_shape* s) {
    sa::Shape r;
    r.batch = s->batch;
    r.T = s->T;
    r.heads = s->heads;
    r.kv_heads = s->kv_heads;
    r.causal = s->causal;
    r.seqlens = s->seqlens;
    r.block_order = s->block_order;
    r.v_rows = s->v_rows;
    return r;
}

sa_status from_hip(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_DEVICE; }

sa_shape batch1_causal(int T, int heads, int kv_heads) {
    sa_shape s;
    s.batch = 1;
    s.T = T;
    s.heads = heads;
    s.kv_heads = kv_heads;
    s.causal = 1;
    s.seqlens = nullptr;
    s.block_order = 0;
    s.v_rows = 0;
    return s;
}

}  // namespace

extern "C" {

sa_status sa_check_shape(const sa_shape* shape) {
    if (!shape) return SA_ERR_NULL;
    const sa_shape& s = *shape;
    if (s.batch < 1 || s.T < 64 || s.T % 64 != 0 || s.T > (1 << 20)) return SA_ERR_SHAPE;
    if (s.heads < 1 || s.kv_heads < 1 || s.heads % s.kv_heads != 0 || s.heads > 65535) return SA_ERR_SHAPE;
    if ((long long)s.batch * s.heads > (1ll << 24)) return SA_ERR_SHAPE;
    if ((s.causal != 0 && s.causal != 1) || (s.block_order != 0 && s.block_order != 1) ||
        (s.v_rows != 0 && s.v_rows != 1))
        return SA_ERR_SHAPE;
    if (s.seqlens && ((uintptr_t)s.seqlens & 3u)) return SA_ERR_ALIGN;
    const sa::Shape sh = to_shape(shape);
    const size_t lim = (size_t)INT_MAX;
    if (sa::forward_blocks(sh) > lim || sa::row_terms_blocks(sh) > lim || sa::key_pass_blocks(sh) > lim ||
        sa::dq_pass_blocks(sh) > lim || sa::query_pass_blocks(sh) > lim)
        return SA_ERR_SHAPE;
    return SA_OK;
}

sa_status sa_forward_ex(const sa_shape* shape, const void* Q, const void* K, const void* Vt, void* O, float* L,
                        float c, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({Q, K, Vt, O, L})) != SA_OK) return st;
    if (!scale_ok(c)) return SA_ERR_ARGUMENT;
    return from_hip(sa::launch_forward(to_shape(shape), Q, K, Vt, O, L, c, (hipStream_t)stream));
}

sa_status sa_forward(const void* Q, const void* K, const void* Vt, void* O, float* L, float c, int T, int heads,
                     int kv_heads, void* stream) {
    sa_shape s = batch1_causal(T, heads, kv_heads);
    return sa_forward_ex(&s, Q, K, Vt, O, L, c, stream);
}

size_t sa_backward_workspace_bytes(const sa_shape* shape) {
    if (sa_check_shape(shape) != SA_OK) return 0;
    const sa::Shape sh = to_shape(shape);
    return (size_t)sh.batch * sh.heads * sa::ds_tiles_per_head(sh) * sa::kDsTileBytes;
}

sa_status sa_row_terms(const sa_shape* shape, const void* dO, const void* O, float* D, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, D})) != SA_OK) return st;
    return from_hip(sa::launch_row_terms(to_shape(shape), dO, O, D, (hipStream_t)stream));
}

sa_status sa_key_pass(const sa_shape* shape, const void* Q, const void* K, const void* Vt, const void* dO,
                      const float* L, const float* D, void* dS, size_t dS_bytes, float c, float s, float* dK,
                      float* dVt, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({Q, K, Vt, dO, L, D, dK, dVt})) != SA_OK) return st;
    if (dS) {  // NULL: the two-launch backward's key launch, nothing stored
        if ((st = check_ptrs({dS})) != SA_OK) return st;
        if (dS_bytes < sa_backward_workspace_bytes(shape)) return SA_ERR_WORKSPACE;
    }
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    return from_hip(sa::launch_key_pass(to_shape(shape), Q, K, Vt, dO, L, D, dS, c, s, dK, dVt,
                                        (hipStream_t)stream));
}

sa_status sa_dq_pass(const sa_shape* shape, const void* K, const void* dS, size_t dS_bytes, float s, float* dQ,
                     void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({K, dS, dQ})) != SA_OK) return st;
    if (dS_bytes < sa_backward_workspace_bytes(shape)) return SA_ERR_WORKSPACE;
    if (!scale_ok(s)) return SA_ERR_ARGUMENT;
    return from_hip(sa::launch_dq_pass(to_shape(shape), K, dS, s, dQ, (hipStream_t)stream));
}

sa_status sa_dq_pass_rotated(const sa_shape* shape, const void* K, const void* dS, size_t dS_bytes, float s,
                             const float* cos_t, const float* sin_t, void* dqkv, int width, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({K, dS, cos_t, sin_t, dqkv})) != SA_OK) return st;
    if (dS_bytes < sa_backward_workspace_bytes(shape)) return SA_ERR_WORKSPACE;
    if (!scale_ok(s)) return SA_ERR_ARGUMENT;
    if (width % 8 != 0 || (long long)width < 64ll * shape->heads) return SA_ERR_ARGUMENT;
    return from_hip(sa::launch_dq_pass_rotated(to_shape(shape), K, dS, s, cos_t, sin_t, dqkv, width,
                                               (hipStream_t)stream));
}

sa_status sa_backward_projection(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D,
                                 void* dS, size_t dS_bytes, const void* Q, const void* K, const void* Vt,
                                 float c, float s, float* dQ32, void* dQ16, float* dK32, void* dK16,
                                 float* dV32, void* dV16, int width, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, D, dS, Q, K, Vt, dQ32, dQ16, dK32, dK16, dV32, dV16})) != SA_OK) return st;
    if (dS_bytes < sa_backward_workspace_bytes(shape)) return SA_ERR_WORKSPACE;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    if (width % 8 != 0 || (long long)width < 64ll * shape->heads) return SA_ERR_ARGUMENT;
    const sa::Shape sh = to_shape(shape);
    hipStream_t strm = (hipStream_t)stream;
    const sa::ProjectionOut q{dQ32, (uint16_t*)dQ16, width}, k{dK32, (uint16_t*)dK16, width},
        v{dV32, (uint16_t*)dV16, width};
    if ((st = from_hip(sa::launch_row_terms(sh, dO, O, D, strm))) != SA_OK) return st;
    if ((st = from_hip(sa::launch_key_pass_projection(sh, Q, K, Vt, dO, L, D, dS, c, s, k, v, strm))) != SA_OK)
        return st;
    return from_hip(sa::launch_dq_pass_projection(sh, K, dS, s, q, strm));
}

sa_status sa_backward_ex(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D, void* dS,
                         size_t dS_bytes, const void* Q, const void* K, const void* Vt, float c, float s,
                         float* dQ, float* dK, float* dVt, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, D, dS, Q, K, Vt, dQ, dK, dVt})) != SA_OK) return st;
    if (dS_bytes < sa_backward_workspace_bytes(shape)) return SA_ERR_WORKSPACE;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    const sa::Shape sh = to_shape(shape);
    hipStream_t strm = (hipStream_t)stream;
    if ((st = from_hip(sa::launch_row_terms(sh, dO, O, D, strm))) != SA_OK) return st;
    if ((st = from_hip(sa::launch_key_pass(sh, Q, K, Vt, dO, L, D, dS, c, s, dK, dVt, strm))) != SA_OK) return st;
    return from_hip(sa::launch_dq_pass(sh, K, dS, s, dQ, strm));
}

size_t sa_backward_chunked_min_bytes(const sa_shape* shape) {
    if (sa_check_shape(shape) != SA_OK) return 0;
    return sa::min_chunk_bytes(to_shape(shape));
}

sa_status sa_backward_chunked(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D,
                              void* dS, size_t dS_bytes, const void* Q, const void* K, const void* Vt, float c,
                              float s, float* dQ, float* dK, float* dVt, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, D, dS, Q, K, Vt, dQ, dK, dVt})) != SA_OK) return st;
    if (dS_bytes < sa_backward_chunked_min_bytes(shape)) return SA_ERR_WORKSPACE;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    const sa::Shape sh = to_shape(shape);
    hipStream_t strm = (hipStream_t)stream;
    if ((st = from_hip(sa::launch_row_terms(sh, dO, O, D, strm))) != SA_OK) return st;
    return from_hip(sa::launch_key_dq_chunked(sh, Q, K, Vt, dO, L, D, dS, dS_bytes, c, s, dQ, dK, dVt, strm));
}

sa_status sa_backward(const void* dO, const void* O, const float* L, float* D, void* dS, size_t dS_bytes,
                      const void* Q, const void* K, const void* Vt, float c, float s, int T, int heads,
                      int kv_heads, float* dQ, float* dK, float* dVt, void* stream) {
    sa_shape sh = batch1_causal(T, heads, kv_heads);
    return sa_backward_ex(&sh, dO, O, L, D, dS, dS_bytes, Q, K, Vt, c, s, dQ, dK, dVt, stream);
}

sa_status sa_query_pass(const sa_shape* shape, const void* dO, const void* O, const float* L, const void* Q,
                        const void* K, const void* Vt, float c, float s, float* D, float* dQ, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, Q, K, Vt, D, dQ})) != SA_OK) return st;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    return from_hip(sa::launch_query_pass(to_shape(shape), dO, O, L, Q, K, Vt, c, s, D, dQ, (hipStream_t)stream));
}

sa_status sa_backward_two_pass(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D,
                               const void* Q, const void* K, const void* Vt, float c, float s, float* dQ,
                               float* dK, float* dVt, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, D, Q, K, Vt, dQ, dK, dVt})) != SA_OK) return st;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    const sa::Shape sh = to_shape(shape);
    hipStream_t strm = (hipStream_t)stream;
    if ((st = from_hip(sa::launch_query_pass(sh, dO, O, L, Q, K, Vt, c, s, D, dQ, strm))) != SA_OK) return st;
    return from_hip(sa::launch_key_pass(sh, Q, K, Vt, dO, L, D, nullptr, c, s, dK, dVt, strm));
}

sa_status sa_backward_two_pass_projection(const sa_shape* shape, const void* dO, const void* O, const float* L,
                                          float* D, const void* Q, const void* K, const void* Vt, float c, float s,
                                          float* dQ32, void* dQ16, float* dK32, void* dK16, float* dV32, void* dV16,
                                          int width, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    if ((st = check_ptrs({dO, O, L, D, Q, K, Vt, dQ32, dQ16, dK32, dK16, dV32, dV16})) != SA_OK) return st;
    if (!scale_ok(c) || !scale_ok(s)) return SA_ERR_ARGUMENT;
    if (width % 8 != 0 || (long long)width < 64ll * shape->heads) return SA_ERR_ARGUMENT;
    const sa::Shape sh = to_shape(shape);
    hipStream_t strm = (hipStream_t)stream;
    const sa::ProjectionOut q{dQ32, (uint16_t*)dQ16, width}, k{dK32, (uint16_t*)dK16, width},
        v{dV32, (uint16_t*)dV16, width};
    if ((st = from_hip(sa::launch_query_pass_projection(sh, dO, O, L, Q, K, Vt, c, s, D, q, strm))) != SA_OK)
        return st;
    return from_hip(sa::launch_key_pass_projection(sh, Q, K, Vt, dO, L, D, nullptr, c, s, k, v, strm));
}

const char* sa_status_string(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_SHAPE: return "shape fails admission (T multiple of 64, heads divisible by kv_heads, limits)";
        case SA_ERR_NULL: return "a required pointer is NULL";
        case SA_ERR_ALIGN: return "a pointer is not 16-byte aligned (seqlens: 4-byte)";
        case SA_ERR_WORKSPACE: return "dS workspace too small (sa_backward_workspace_bytes; sa_backward_chunked_min_bytes for the chunked backward)";
        case SA_ERR_ARGUMENT: return "scale c or s is not finite and positive, or a bad projection width";
        case SA_ERR_DEVICE: return "a HIP kernel launch failed";
        case SA_ERR_TOO_LARGE: return "the dS workspace exceeds the library's static scratch (SA_STATIC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
