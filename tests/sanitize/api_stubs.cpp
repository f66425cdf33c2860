// Host-only stand-ins for the kernel launchers behind the C ABI, so that
// csrc/sa_api.cpp (admission, argument checks, launch sequencing) and the
// chunk planning of the chunked backward can be built and run with
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// Every launcher records its call and returns hipSuccess; nothing touches a
// device.  Test infrastructure: built by tests/test_sanitizers.py only.
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "sa_internal.h"

std::vector<std::string> g_calls;
std::vector<sa::Chunk> g_chunks;

namespace sa {

size_t forward_blocks(const Shape& sh) { return (size_t)sh.batch * sh.heads * (size_t)((sh.T + 255) / 256); }
size_t row_terms_blocks(const Shape& sh) { return ((size_t)sh.batch * sh.heads * sh.T + 31) / 32; }
size_t key_pass_blocks(const Shape& sh) { return (size_t)sh.batch * sh.kv_heads * (size_t)(sh.T / 64); }
size_t dq_pass_blocks(const Shape& sh) { return (size_t)sh.batch * sh.heads * (size_t)((sh.T + 255) / 256); }
size_t query_pass_blocks(const Shape& sh) { return (size_t)sh.batch * sh.heads * (size_t)((sh.T + 255) / 256); }

hipError_t launch_forward(const Shape&, const void*, const void*, const void*, void*, float*, float, hipStream_t) {
    g_calls.push_back("forward");
    return hipSuccess;
}
hipError_t launch_row_terms(const Shape&, const void*, const void*, float*, hipStream_t) {
    g_calls.push_back("row_terms");
    return hipSuccess;
}
hipError_t launch_key_pass(const Shape&, const void*, const void*, const void*, const void*, const float*,
                           const float*, void* dS, float, float, float*, float*, hipStream_t) {
    g_calls.push_back(dS ? "key_pass" : "key_pass_no_ds");
    return hipSuccess;
}
hipError_t launch_dq_pass(const Shape&, const void*, const void*, float, float*, hipStream_t) {
    g_calls.push_back("dq_pass");
    return hipSuccess;
}
size_t min_chunk_bytes(const Shape& sh) { return largest_block_bytes(sh); }
hipError_t launch_key_dq_chunked(const Shape& sh, const void*, const void*, const void*, const void*, const float*,
                                 const float*, void*, size_t ws_bytes, float, float, float*, float*, float*,
                                 hipStream_t) {
    if (ws_bytes < min_chunk_bytes(sh)) return hipErrorInvalidValue;
    int q_hi = sh.T / 64;
    bool first = true;
    while (q_hi > 0) {
        const Chunk ch = next_chunk(sh, q_hi, ws_bytes, first);
        g_chunks.push_back(ch);
        g_calls.push_back("chunk");
        first = false;
        q_hi = ch.q_lo;
    }
    return hipSuccess;
}
hipError_t launch_dq_pass_rotated(const Shape&, const void*, const void*, float, const float*, const float*, void*,
                                  int, hipStream_t) {
    g_calls.push_back("dq_pass_rotated");
    return hipSuccess;
}
hipError_t launch_key_pass_projection(const Shape&, const void*, const void*, const void*, const void*,
                                      const float*, const float*, void* dS, float, float, const ProjectionOut&,
                                      const ProjectionOut&, hipStream_t) {
    g_calls.push_back(dS ? "key_pass_projection" : "key_pass_projection_no_ds");
    return hipSuccess;
}
hipError_t launch_dq_pass_projection(const Shape&, const void*, const void*, float, const ProjectionOut&,
                                     hipStream_t) {
    g_calls.push_back("dq_pass_projection");
    return hipSuccess;
}
hipError_t launch_query_pass_projection(const Shape&, const void*, const void*, const float*, const void*,
                                        const void*, const void*, float, float, float*, const ProjectionOut&,
                                        hipStream_t) {
    g_calls.push_back("query_pass_projection");
    return hipSuccess;
}
hipError_t launch_query_pass(const Shape&, const void*, const void*, const float*, const void*, const void*,
                             const void*, float, float, float*, float*, hipStream_t) {
    g_calls.push_back("query_pass");
    return hipSuccess;
}

}  // namespace sa
