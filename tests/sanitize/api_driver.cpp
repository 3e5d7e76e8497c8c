// Drives every entry point of the C front end through its validation paths
// (invalid and valid arguments) under ASan/UBSan.  Pointers are fake,
// well-aligned addresses that validation never dereferences; the launchers
// are stubs (api_stubs.cpp).  Exits non-zero on a wrong status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "attnres.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static void* P(uintptr_t k) { return reinterpret_cast<void*>(k << 20); }
static float* F(uintptr_t k) { return static_cast<float*>(P(k)); }

int main() {
    const attnres_dtype B = ATTNRES_BF16, S32 = ATTNRES_F32;
    // full forward
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 64, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_OK);
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 12, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_ALIGN);
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 64, F(2), 5, 9, 1e-6f, nullptr, 0, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 64, F(2), 0, 9, -1.f, nullptr, 0, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_full_fwd(nullptr, B, 9, 16, 64, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_full_fwd(P(1), B, 9, (int64_t)1 << 23, 64, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), B,
                            nullptr, nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_UNSUPPORTED);
    {   // a call the stubs split between two launches (leading reads, then the rest)
        const int before = g_launches;
        EXPECT(attnres_full_fwd(P(1), B, 40, 16, 64, F(2), 0, 40, 1e-6f, F(4), 3, P(3), B, F(5),
                                nullptr, nullptr, F(6), nullptr) == ATTNRES_OK);
        EXPECT(g_launches == before + 2);
    }
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 64, F(2), 0, 9, 1e-6f, F(4), 3, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_OK);
    EXPECT(attnres_full_fwd(P(1), B, 9, 16, 64, F(2), 0, 9, 1e-6f, nullptr, 3, P(3), B, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_full_fwd_q(P(1), B, 9, 16, 64, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), S32, nullptr,
                              nullptr) == ATTNRES_OK);
    EXPECT(attnres_query_proj(P(1), B, 3, 16, 64, P(2), B, F(3), nullptr) == ATTNRES_OK);
    EXPECT(attnres_query_proj(P(1), S32, 3, 16, 64, P(2), B, F(3), nullptr) == ATTNRES_ERR_UNSUPPORTED);
    // block forward, both query forms
    EXPECT(attnres_block_fwd(P(1), B, 17, 16, 64, 4, F(2), 0, 17, 1e-6f, P(3), B, nullptr, nullptr,
                             nullptr) == ATTNRES_OK);
    EXPECT(attnres_block_fwd(P(1), B, 17, 16, 64, 0, F(2), 0, 17, 1e-6f, P(3), B, nullptr, nullptr,
                             nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_block_fwd_q(P(1), B, 17, 16, 64, 4, F(2), 3, 14, 1e-6f, P(3), B, nullptr,
                               nullptr) == ATTNRES_OK);
    EXPECT(attnres_block_fwd_q(P(1), B, 17, 16, 64, 4, nullptr, 3, 14, 1e-6f, P(3), B, nullptr,
                               nullptr) == ATTNRES_ERR_INVALID_ARG);
    // model-order phases
    EXPECT(attnres_block_phase1(F(1), 3, 16, 64, P(2), B, F(3), F(4), 4, 1e-6f, F(5), F(6), F(7),
                                P(8), B, F(9), nullptr, nullptr, nullptr) == ATTNRES_OK);
    EXPECT(attnres_block_phase1(F(1), 14, 16, 64, P(2), B, F(3), F(4), 4, 1e-6f, F(5), F(6), F(7),
                                P(8), B, F(9), nullptr, nullptr, nullptr) == ATTNRES_ERR_UNSUPPORTED);
    EXPECT(attnres_block_phase1_q(F(1), 3, 16, 64, nullptr, B, nullptr, F(4), 1, 1e-6f, F(5), F(6),
                                  F(7), nullptr, B, nullptr, nullptr) == ATTNRES_OK);
    EXPECT(attnres_block_phase1_q(F(1), 3, 16, 64, nullptr, B, F(3), F(4), 1, 1e-6f, F(5), F(6),
                                  F(7), nullptr, B, nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_block_phase2(P(1), B, 16, 64, F(2), 1, F(3), F(4), F(5), 1e-6f, P(6), B, nullptr,
                                nullptr, nullptr, nullptr) == ATTNRES_OK);
    EXPECT(attnres_block_phase2_q(P(1), B, 16, 64, F(2), 2, F(3), F(4), F(5), 1e-6f, P(6), B,
                                  nullptr, nullptr) == ATTNRES_ERR_INVALID_ARG);
    // backward with a workspace, with accumulation, without allocation
    const size_t ws = attnres_bwd_workspace_bytes(ATTNRES_BLOCK, 4, 17, 16, 64, 0, 17);
    EXPECT(ws > 0);
    EXPECT(attnres_bwd(ATTNRES_BLOCK, 4, P(1), B, 17, 16, 64, F(2), 0, 17, 1e-6f, P(3), B, P(4),
                       S32, 1, F(5), P(6), ws, nullptr) == ATTNRES_OK);
    EXPECT(attnres_bwd(ATTNRES_BLOCK, 4, P(1), B, 17, 16, 64, F(2), 0, 17, 1e-6f, P(3), B, P(4), B,
                       1, F(5), P(6), ws, nullptr) == ATTNRES_ERR_INVALID_ARG);
    EXPECT(attnres_bwd(ATTNRES_BLOCK, 4, P(1), B, 17, 16, 64, F(2), 0, 17, 1e-6f, P(3), B, P(4), B,
                       0, F(5), P(6), ws - 1, nullptr) == ATTNRES_ERR_WORKSPACE);
    EXPECT(attnres_bwd(ATTNRES_FULL, 1, P(1), B, 5000, 16, 64, F(2), 0, 5000, 1e-6f, P(3), B, P(4),
                       B, 0, F(5), P(6), (size_t)1 << 40, nullptr) == ATTNRES_ERR_UNSUPPORTED);
    EXPECT(attnres_bwd_noalloc(ATTNRES_FULL, 1, P(1), B, 17, 16, 64, F(2), 0, 17, 1e-6f, P(3), B,
                               P(4), B, 0, F(5), nullptr) == ATTNRES_OK);
    EXPECT(attnres_bwd_noalloc(ATTNRES_FULL, 1, P(1), B, 49, 4096, 1024, F(2), 0, 49, 1e-6f, P(3), B,
                               P(4), B, 0, F(5), nullptr) == ATTNRES_ERR_UNSUPPORTED);
    // host-only index table into a real buffer, and rejects
    std::vector<int32_t> tab(3 * 65);
    EXPECT(attnres_block_index_table(65, 8, 0, 65, tab.data()) == ATTNRES_OK);
    EXPECT(tab[3 * 64 + 0] == 8 && tab[3 * 64 + 1] == 65 && tab[3 * 64 + 2] == 65);
    EXPECT(attnres_block_index_table(65, 8, 1, 65, tab.data()) == ATTNRES_ERR_INVALID_ARG);
    // status strings and the thread-local error text
    for (int s = -1; s <= 6; ++s) EXPECT(std::strlen(attnres_status_string(s)) > 0);
    std::string other;
    std::thread th([&] {
        attnres_full_fwd(P(1), B, 9, 16, 12, F(2), 0, 9, 1e-6f, nullptr, 0, P(3), B, nullptr,
                         nullptr, nullptr, nullptr, nullptr);
        other = attnres_last_error();
    });
    th.join();
    attnres_block_index_table(65, 8, 0, 65, tab.data());
    EXPECT(!other.empty() && std::strlen(attnres_last_error()) == 0);
    EXPECT(g_launches > 0);
    std::printf("api driver: %d failures, %d stub launches\n", failures, g_launches);
    return failures == 0 ? 0 : 1;
}
