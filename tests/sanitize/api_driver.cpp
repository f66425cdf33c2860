// Calls every C ABI entry point of csrc/sa_api.cpp, built with AddressSanitizer
// and UndefinedBehaviorSanitizer against host-only launcher stand-ins
// (api_stubs.cpp): good and bad shapes, NULL and misaligned pointers, bad
// scales, short workspaces, and, for accepted calls, the launch sequence each
// entry point issues.  The chunked backward's plan is checked to cover every
// query tile once, from the last rows down, each chunk within the workspace.
// Test infrastructure: built and run by tests/test_sanitizers.py only.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "sa.h"
#include "sa_internal.h"

extern std::vector<std::string> g_calls;
extern std::vector<sa::Chunk> g_chunks;

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAILED: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static std::string calls() {
    std::string r;
    for (auto& c : g_calls) r += c + ",";
    g_calls.clear();
    return r;
}

static sa_shape shape(int B, int T, int H, int KV, int causal) {
    sa_shape s;
    memset(&s, 0, sizeof s);
    s.batch = B; s.T = T; s.heads = H; s.kv_heads = KV; s.causal = causal;
    return s;
}

static void check_plan(const sa_shape& s, size_t ws) {
    const sa::Shape sh{s.batch, s.T, s.heads, s.kv_heads, s.causal, nullptr, 0, 0};
    g_chunks.clear();
    void* p = (void*)0x10000;
    float* f = (float*)0x10000;
    sa_status st = sa_backward_chunked(&s, p, p, f, f, p, ws, p, p, p, 0.18f, 0.125f, f, f, f, nullptr);
    if (ws < sa_backward_chunked_min_bytes(&s)) {
        EXPECT(st == SA_ERR_WORKSPACE);
        EXPECT(g_chunks.empty());
        g_calls.clear();
        return;
    }
    EXPECT(st == SA_OK);
    EXPECT(!g_chunks.empty());
    int expect_hi = s.T / 64;
    for (size_t i = 0; i < g_chunks.size(); ++i) {
        const sa::Chunk& c = g_chunks[i];
        EXPECT(c.q_hi == expect_hi);
        EXPECT(c.q_lo < c.q_hi && c.q_lo % 2 == 0);
        EXPECT(c.accumulate == (i == 0 ? 0 : 1));
        EXPECT(c.tile0 == sa::ds_row_start(sh, c.q_lo));
        EXPECT(sa::chunk_bytes(sh, c.q_lo, c.q_hi) <= ws);
        EXPECT((size_t)c.tph * s.batch * s.heads * sa::kDsTileBytes == sa::chunk_bytes(sh, c.q_lo, c.q_hi));
        expect_hi = c.q_lo;
    }
    EXPECT(expect_hi == 0);
    if (ws >= sa_backward_workspace_bytes(&s)) EXPECT(g_chunks.size() == 1);
    g_calls.clear();
}

int main() {
    void* p = (void*)0x10000;
    void* mis = (void*)0x10004;
    float* f = (float*)0x10000;
    const float c = 0.18033688f, s = 0.125f;
    sa_shape sh = shape(2, 320, 4, 2, 1);
    EXPECT(sa_check_shape(&sh) == SA_OK);
    const size_t ws = sa_backward_workspace_bytes(&sh);
    EXPECT(ws == (size_t)2 * 4 * 15 * 64 * 64 * 2);

    EXPECT(sa_forward_ex(&sh, p, p, p, p, f, c, nullptr) == SA_OK && calls() == "forward,");
    EXPECT(sa_forward(p, p, p, p, f, c, 320, 4, 2, nullptr) == SA_OK && calls() == "forward,");
    EXPECT(sa_backward_ex(&sh, p, p, f, f, p, ws, p, p, p, c, s, f, f, f, nullptr) == SA_OK &&
           calls() == "row_terms,key_pass,dq_pass,");
    EXPECT(sa_backward_ex(&sh, p, p, f, f, p, ws - 1, p, p, p, c, s, f, f, f, nullptr) == SA_ERR_WORKSPACE);
    EXPECT(sa_backward(p, p, f, f, p, ws / 2 - 1, p, p, p, c, s, 320, 4, 2, f, f, f, nullptr) == SA_ERR_WORKSPACE);
    EXPECT(calls() == "");
    EXPECT(sa_backward(p, p, f, f, p, ws / 2, p, p, p, c, s, 320, 4, 2, f, f, f, nullptr) == SA_OK &&
           calls() == "row_terms,key_pass,dq_pass,");
    EXPECT(calls() == "");
    EXPECT(sa_row_terms(&sh, p, p, f, nullptr) == SA_OK && calls() == "row_terms,");
    EXPECT(sa_key_pass(&sh, p, p, p, p, f, f, nullptr, 0, c, s, f, f, nullptr) == SA_OK &&
           calls() == "key_pass_no_ds,");
    EXPECT(sa_dq_pass(&sh, p, p, ws, s, f, nullptr) == SA_OK && calls() == "dq_pass,");
    EXPECT(sa_query_pass(&sh, p, p, f, p, p, p, c, s, f, f, nullptr) == SA_OK && calls() == "query_pass,");
    EXPECT(sa_backward_two_pass(&sh, p, p, f, f, p, p, p, c, s, f, f, f, nullptr) == SA_OK &&
           calls() == "query_pass,key_pass_no_ds,");
    EXPECT(sa_dq_pass_rotated(&sh, p, p, ws, s, f, f, p, 512, nullptr) == SA_OK && calls() == "dq_pass_rotated,");
    EXPECT(sa_dq_pass_rotated(&sh, p, p, ws, s, f, f, p, 100, nullptr) == SA_ERR_ARGUMENT);
    EXPECT(sa_backward_projection(&sh, p, p, f, f, p, ws, p, p, p, c, s, f, p, f, p, f, p, 512, nullptr) == SA_OK &&
           calls() == "row_terms,key_pass_projection,dq_pass_projection,");
    EXPECT(sa_backward_two_pass_projection(&sh, p, p, f, f, p, p, p, c, s, f, p, f, p, f, p, 512, nullptr) ==
               SA_OK &&
           calls() == "query_pass_projection,key_pass_projection_no_ds,");

    // rejections, before anything is launched
    EXPECT(sa_forward_ex(&sh, p, p, p, nullptr, f, c, nullptr) == SA_ERR_NULL);
    EXPECT(sa_forward_ex(&sh, p, p, mis, p, f, c, nullptr) == SA_ERR_ALIGN);
    EXPECT(sa_forward_ex(&sh, p, p, p, p, f, -c, nullptr) == SA_ERR_ARGUMENT);
    EXPECT(sa_forward_ex(&sh, p, p, p, p, f, 1.0f / 0.0f, nullptr) == SA_ERR_ARGUMENT);
    EXPECT(sa_backward_ex(&sh, p, p, f, f, p, ws, p, p, p, c, s, f, f, (float*)mis, nullptr) == SA_ERR_ALIGN);
    sa_shape bad = shape(1, 100, 4, 2, 1);
    EXPECT(sa_check_shape(&bad) == SA_ERR_SHAPE && sa_backward_workspace_bytes(&bad) == 0);
    bad = shape(1, 128, 3, 2, 1);
    EXPECT(sa_check_shape(&bad) == SA_ERR_SHAPE);
    bad = shape(1, 128, 4, 2, 2);
    EXPECT(sa_check_shape(&bad) == SA_ERR_SHAPE);
    bad = shape(1 << 20, 128, 64, 64, 1);
    EXPECT(sa_check_shape(&bad) == SA_ERR_SHAPE);   /* batch * heads past 2^24 */
    EXPECT(sa_check_shape(nullptr) == SA_ERR_NULL);
    sa_shape odd = sh;
    odd.seqlens = (const int32_t*)0x10002;
    EXPECT(sa_check_shape(&odd) == SA_ERR_ALIGN);
    EXPECT(calls() == "");
    for (int st = -1; st <= 8; ++st) EXPECT(sa_status_string(st) != nullptr && strlen(sa_status_string(st)) > 0);

    // the chunked backward's plan, causal and full, odd and even tile counts, many workspace sizes
    const sa_shape plans[] = {shape(2, 320, 4, 2, 1), shape(1, 384, 2, 1, 1), shape(1, 320, 2, 2, 0),
                              shape(3, 1024, 8, 2, 1), shape(1, 64, 1, 1, 1)};
    for (const sa_shape& ps : plans) {
        const size_t least = sa_backward_chunked_min_bytes(&ps), all = sa_backward_workspace_bytes(&ps);
        check_plan(ps, least - 1);
        for (size_t w = least; w < all + 8192 * 8; w += (all - least) / 7 + 8192) check_plan(ps, w);
        check_plan(ps, all);
    }
    printf("%s\n", fails ? "api-sanitize: failures" : "api-sanitize: ok");
    return fails != 0;
}
