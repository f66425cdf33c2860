// sa_static.hip -- the split backward with its dS workspace in a static
// device array owned by the library, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels are the chunked split backward's own (as many
// query rows per chunk as the array holds); only the workspace differs.
//
// The array lives for the whole process on every GPU the library runs on
// (each GPU holds its own copy at its own address).  In host code its name is
// only a stand-in: its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and that address is what the
// kernels receive.  Every call on one GPU shares that GPU's array, so calls
// that overlap on one GPU (other streams, other threads) race.  Nothing in it
// has to start at zero: the key pass writes every dS element the dQ pass
// reads, exact zeros where masked.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <mutex>

#include "sa.h"
#include "sa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// The scratch array's address on the current device, looked up on the first
// call on that device.  NULL if the lookup fails.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" sa_status sa_backward_static(const sa_shape* shape, const void* dO, const void* O, const float* L,
                                        float* D, const void* Q, const void* K, const void* Vt, float c, float s,
                                        float* dQ, float* dK, float* dVt, void* stream) {
    sa_status st = sa_check_shape(shape);
    if (st != SA_OK) return st;
    const void* ptrs[] = {dO, O, L, D, Q, K, Vt, dQ, dK, dVt};
    for (const void* p : ptrs)
        if (!p) return SA_ERR_NULL;
    for (const void* p : ptrs)
        if (!aligned16(p)) return SA_ERR_ALIGN;
    if (!(std::isfinite(c) && c > 0.0f) || !(std::isfinite(s) && s > 0.0f)) return SA_ERR_ARGUMENT;
    if (sa_backward_chunked_min_bytes(shape) > (size_t)SA_STATIC_SCRATCH_BYTES) return SA_ERR_TOO_LARGE;
    void* ws = scratch_on_current_device();
    if (!ws) return SA_ERR_DEVICE;
    sa::Shape sh;
    sh.batch = shape->batch;
    sh.T = shape->T;
    sh.heads = shape->heads;
    sh.kv_heads = shape->kv_heads;
    sh.causal = shape->causal;
    sh.seqlens = shape->seqlens;
    sh.block_order = shape->block_order;
    sh.v_rows = shape->v_rows;
    hipStream_t strm = (hipStream_t)stream;
    if (sa::launch_row_terms(sh, dO, O, D, strm) != hipSuccess) return SA_ERR_DEVICE;
    if (sa::launch_key_dq_chunked(sh, Q, K, Vt, dO, L, D, ws, SA_STATIC_SCRATCH_BYTES, c, s, dQ, dK, dVt, strm) !=
        hipSuccess)
        return SA_ERR_DEVICE;
    return SA_OK;
}
