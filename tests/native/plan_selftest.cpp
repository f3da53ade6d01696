// plan_selftest.cpp -- a stand-alone driver of the library's host-only entry
// points for sanitizer builds (host code built with AddressSanitizer and
// UndefinedBehaviorSanitizer): plans many shapes through mlp_chain_plan and
// checks the planner's contract (one K split for every policy, no empty K
// part, tiles covering the matrices, the tuned table and the rules), then
// feeds every entry point arguments it must refuse without touching a
// device.  Exits 0 when all hold.  Test infrastructure: built and run by
// tests/test_sanitizers.py.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mlp_chain.h"

static int fails = 0;
#define CHECK(c, ...)                     \
    do {                                  \
        if (!(c)) {                       \
            fprintf(stderr, __VA_ARGS__); \
            fputc('\n', stderr);          \
            ++fails;                      \
        }                                 \
    } while (0)

int main() {
    const int64_t Ms[] = {1, 2, 15, 16, 17, 63, 64, 100, 128, 255, 256, 257, 512, 777, 1024, 2048, 4096, 8192};
    const int64_t HI[][2] = {{512, 2048}, {12288, 6144}, {8192, 2752}, {8192, 3584}, {8192, 8192}, {328, 456}, {8, 8},
                             {1032, 776}};
    const int cuss[] = {256, -256, 80, 304, 8, -8};
    int64_t plan[3][14];
    long n = 0;
    for (int64_t M : Ms)
        for (auto& hi : HI)
            for (int act = 0; act < 3; ++act)
                for (int cus : cuss) {
                    const int64_t H = hi[0], I = hi[1];
                    for (int pol = 0; pol < 3; ++pol) {
                        memset(plan[pol], 0xff, sizeof plan[pol]);
                        CHECK(mlp_chain_plan(M, H, I, act, pol, cus, plan[pol], 14) == MLP_OK, "plan failed: %s",
                              mlp_chain_last_error());
                        const int64_t* p = plan[pol];
                        const int64_t S1 = p[1], S2 = p[2], BM = p[3], BN1 = p[4], BN2 = p[5], Mt = p[6];
                        const int64_t N1t = p[7], N2t = p[8], T1 = p[9], T2 = p[10], k1 = p[11], k2 = p[12];
                        const int64_t n1 = (H + 63) / 64, n2 = (I + 63) / 64;
                        CHECK(S1 >= 1 && (S1 - 1) * k1 < n1 && n1 <= S1 * k1, "GEMM1 K parts %lld x %lld of %lld",
                              (long long)S1, (long long)k1, (long long)n1);
                        CHECK(S2 >= 1 && (S2 - 1) * k2 < n2 && n2 <= S2 * k2, "GEMM2 K parts");
                        CHECK(Mt * BM >= M && (Mt - 1) * BM < M, "row blocks");
                        CHECK(N1t * BN1 >= I && N2t * BN2 >= H, "column blocks");
                        CHECK(T1 == Mt * N1t && T2 == Mt * N2t, "tile counts");
                        CHECK(p[13] == 0 || p[13] == 1, "tuned flag");
                        if (cus < 0) CHECK(p[13] == 0, "rules-only plan reported as tuned");
                        ++n;
                    }
                    CHECK(plan[0][1] == plan[1][1] && plan[0][1] == plan[2][1] && plan[0][2] == plan[1][2] &&
                              plan[0][2] == plan[2][2],
                          "policies split K differently: M=%lld H=%lld I=%lld act=%d cus=%d", (long long)M,
                          (long long)H, (long long)I, act, cus);
                }
    // arguments every entry point must refuse without a device
    int64_t a[14];
    CHECK(mlp_chain_plan(0, 512, 512, 1, 2, 256, a, 14) == MLP_EINVAL, "M = 0 planned");
    CHECK(mlp_chain_plan(4, 500, 512, 1, 2, 256, a, 14) == MLP_EINVAL, "H not a multiple of 8 planned");
    CHECK(mlp_chain_plan(4, 512, 512, 3, 2, 256, a, 14) == MLP_EINVAL, "act 3 planned");
    CHECK(mlp_chain_plan(4, 512, 512, 1, 3, 256, a, 14) == MLP_EINVAL, "policy 3 planned");
    CHECK(mlp_chain_plan(4, 512, 512, 1, 2, 4, a, 14) == MLP_EINVAL, "4 CUs planned");
    CHECK(mlp_chain_plan(4, 512, 512, 1, 2, 256, nullptr, 14) == MLP_EINVAL, "NULL plan array");
    CHECK(mlp_chain_plan(1 << 30, 8192, 8192, 0, 2, 256, a, 14) == MLP_EINVAL, "oversized M planned");
    CHECK(mlp_chain_create(0, 512, 512, 1, 0, 2) == nullptr && strstr(mlp_chain_last_error(), "sizes"),
          "create accepted M = 0");
    CHECK(mlp_chain_create_layers(4, 512, 512, 1, 0, 2, 0) == nullptr, "create accepted 0 layers");
    CHECK(mlp_chain_run(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == MLP_EINVAL, "run NULL");
    CHECK(mlp_chain_run_layers(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == MLP_EINVAL, "run_layers NULL");
    CHECK(mlp_chain_status(nullptr) == MLP_EINVAL && mlp_chain_destroy(nullptr) == MLP_OK, "NULL handle");
    CHECK(mlp_chain_info(nullptr, a, 14) == MLP_EINVAL, "info NULL");
    CHECK(mlp_chain_run_noalloc(0, 8, 8, 0, 0, 0, a, a, a, a, nullptr, nullptr) == MLP_EINVAL, "noalloc M = 0");
    printf("plan selftest: %ld plans, %d failures\n", n, fails);
    return fails ? 1 : 0;
}
