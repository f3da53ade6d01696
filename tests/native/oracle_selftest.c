/*
 * oracle_selftest.c -- a stand-alone driver of the CPU oracle (mlp_oracle.c)
 * for sanitizer builds (gcc -fsanitize=address,undefined): it runs the chain
 * on small shapes of every activation and dtype, ragged and tiny, checks
 * closed-form properties that need no second implementation (zero X gives
 * zero, identity W2 gives the intermediate, exact integers give int64
 * products), exercises the argument checks, and exits 0 when all hold.
 * Test infrastructure: built and run by tests/test_sanitizers.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_mlp_chain(const uint16_t* x, const uint16_t* w1, const uint16_t* w2, uint16_t* t, uint16_t* y,
                     int64_t M, int64_t H, int64_t I, int act, int dtype, int nthreads);
void oracle_widen(const uint16_t* in, float* out, int64_t n, int dtype);
void oracle_round(const float* in, uint16_t* out, int64_t n, int dtype);

static uint32_t rng = 12345u;
static uint32_t next(void) {
    rng = rng * 1664525u + 1013904223u;
    return rng >> 8;
}

/* bits of a small value in [-r, r] / scale, rounded by the oracle itself */
static uint16_t val(int dtype, int r, float scale) {
    float v = (float)((int)(next() % (uint32_t)(2 * r + 1)) - r) / scale;
    uint16_t b;
    oracle_round(&v, &b, 1, dtype);
    return b;
}

static int fails = 0;
#define CHECK(c, ...)                         \
    do {                                      \
        if (!(c)) {                           \
            fprintf(stderr, __VA_ARGS__);     \
            fputc('\n', stderr);              \
            ++fails;                          \
        }                                     \
    } while (0)

static void one_case(int64_t M, int64_t H, int64_t I, int act, int dtype) {
    const int64_t g = act == 2 ? 2 : 1;
    uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(M * H));
    uint16_t* w1 = malloc(sizeof(uint16_t) * (size_t)(H * g * I));
    uint16_t* w2 = malloc(sizeof(uint16_t) * (size_t)(I * H));
    uint16_t* t = malloc(sizeof(uint16_t) * (size_t)(M * I));
    uint16_t* y = malloc(sizeof(uint16_t) * (size_t)(M * H));
    uint16_t* y2 = malloc(sizeof(uint16_t) * (size_t)(M * H));
    float* f = malloc(sizeof(float) * (size_t)(M * (I > H ? I : H)));
    for (int64_t i = 0; i < M * H; ++i) x[i] = val(dtype, 8, 4.0f);
    for (int64_t i = 0; i < H * g * I; ++i) w1[i] = val(dtype, 8, 16.0f);
    for (int64_t i = 0; i < I * H; ++i) w2[i] = val(dtype, 8, 16.0f);
    CHECK(oracle_mlp_chain(x, w1, w2, t, y, M, H, I, act, dtype, 0) == 0, "chain failed");
    /* thread count does not change a bit */
    CHECK(oracle_mlp_chain(x, w1, w2, NULL, y2, M, H, I, act, dtype, 1) == 0, "chain (1 thread) failed");
    CHECK(memcmp(y, y2, sizeof(uint16_t) * (size_t)(M * H)) == 0, "thread count changed the output");
    /* zero X gives zero Y (every activation is 0 at 0) */
    memset(x, 0, sizeof(uint16_t) * (size_t)(M * H));
    CHECK(oracle_mlp_chain(x, w1, w2, NULL, y, M, H, I, act, dtype, 0) == 0, "chain failed");
    oracle_widen(y, f, M * H, dtype);
    for (int64_t i = 0; i < M * H; ++i) CHECK(f[i] == 0.0f, "zero X: y[%lld] = %g", (long long)i, f[i]);
    /* identity W2 (I >= H) returns the first H columns of the intermediate */
    if (I >= H) {
        for (int64_t i = 0; i < M * H; ++i) x[i] = val(dtype, 8, 4.0f);
        memset(w2, 0, sizeof(uint16_t) * (size_t)(I * H));
        const float one = 1.0f;
        uint16_t ob;
        oracle_round(&one, &ob, 1, dtype);
        for (int64_t i = 0; i < H; ++i) w2[i * H + i] = ob;
        CHECK(oracle_mlp_chain(x, w1, w2, t, y, M, H, I, act, dtype, 0) == 0, "chain failed");
        /* numerically equal (a -0 in the intermediate sums to +0) */
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < H; ++n) {
                float a, c;
                oracle_widen(&y[m * H + n], &a, 1, dtype);
                oracle_widen(&t[m * I + n], &c, 1, dtype);
                CHECK(a == c, "identity W2: y[%lld,%lld] = %g, t = %g", (long long)m, (long long)n, a, c);
            }
    }
    free(x); free(w1); free(w2); free(t); free(y); free(y2); free(f);
}

static void integer_case(int dtype) {
    /* act none, small integers: the chain equals int64 products rounded */
    const int64_t M = 5, H = 33, I = 17;
    int64_t xi[5 * 33], w1i[33 * 17], w2i[17 * 33];
    uint16_t x[5 * 33], w1[33 * 17], w2[17 * 33], y[5 * 33];
    float fx;
    for (int64_t i = 0; i < M * H; ++i) { xi[i] = (int64_t)(next() % 7) - 3; fx = (float)xi[i]; oracle_round(&fx, &x[i], 1, dtype); }
    for (int64_t i = 0; i < H * I; ++i) { w1i[i] = (int64_t)(next() % 5) - 2; fx = (float)w1i[i]; oracle_round(&fx, &w1[i], 1, dtype); }
    for (int64_t i = 0; i < I * H; ++i) { w2i[i] = (int64_t)(next() % 3) - 1; fx = (float)w2i[i]; oracle_round(&fx, &w2[i], 1, dtype); }
    CHECK(oracle_mlp_chain(x, w1, w2, NULL, y, M, H, I, 0, dtype, 0) == 0, "integer chain failed");
    for (int64_t m = 0; m < M; ++m) {
        float tf[17];
        for (int64_t i = 0; i < I; ++i) {
            int64_t h = 0;
            for (int64_t k = 0; k < H; ++k) h += xi[m * H + k] * w1i[k * I + i];
            const float hf = (float)h;
            uint16_t tb;
            oracle_round(&hf, &tb, 1, dtype);
            oracle_widen(&tb, &tf[i], 1, dtype);
        }
        for (int64_t n = 0; n < H; ++n) {
            int64_t s = 0;
            for (int64_t i = 0; i < I; ++i) s += (int64_t)tf[i] * w2i[i * H + n];
            const float sf = (float)s;
            uint16_t yb;
            oracle_round(&sf, &yb, 1, dtype);
            CHECK(yb == y[m * H + n], "integer chain: y[%lld,%lld]", (long long)m, (long long)n);
        }
    }
}

int main(void) {
    static const int64_t shapes[][3] = {{1, 8, 8}, {3, 17, 40}, {16, 64, 24}, {7, 40, 96}, {2, 1, 1}};
    for (int s = 0; s < 5; ++s)
        for (int act = 0; act < 3; ++act)
            for (int dtype = 0; dtype < 2; ++dtype) one_case(shapes[s][0], shapes[s][1], shapes[s][2], act, dtype);
    integer_case(0);
    integer_case(1);
    /* argument checks */
    uint16_t b[8] = {0};
    CHECK(oracle_mlp_chain(b, b, b, NULL, b, -1, 2, 2, 0, 0, 0) == -1, "negative M accepted");
    CHECK(oracle_mlp_chain(b, b, b, NULL, b, 1, 2, 2, 3, 0, 0) == -1, "bad act accepted");
    CHECK(oracle_mlp_chain(b, b, b, NULL, b, 1, 2, 2, 0, 2, 0) == -1, "bad dtype accepted");
    CHECK(oracle_mlp_chain(NULL, b, b, NULL, b, 1, 2, 2, 0, 0, 0) == -1, "NULL x accepted");
    CHECK(oracle_mlp_chain(b, b, b, NULL, b, 0, 2, 2, 0, 0, 0) == 0, "M = 0 refused");
    printf("oracle selftest: %d failures\n", fails);
    return fails ? 1 : 0;
}
