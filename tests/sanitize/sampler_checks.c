/* The sampler oracle (oracle/sampler.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: full and top-k updates over ragged
 * vocabularies, non-finite rows, stopped canvases, corruption, cross-entropy
 * and canvas initialisation.  Exit code 0 when the runs finish (the
 * sanitizers abort on the first report). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void ora_sample_update(int lock_rule, float theta, float T0, float T1, float tau,
                       int require_stable, int max_steps, uint64_t seed, int step, int B, int N,
                       int V, const float* logits, int32_t* canvas, int32_t* argmax,
                       uint8_t* lock, float* stats, int32_t* stop);
void ora_sample_update_topk(int lock_rule, float theta, float T0, float T1, float tau,
                            int require_stable, int max_steps, uint64_t seed, int step, int K,
                            int B, int N, int V, const float* logits, int32_t* canvas,
                            int32_t* argmax, uint8_t* lock, float* stats, int32_t* stop);
void ora_canvas_init(uint64_t seed, int block, int B, int N, int V, int32_t* canvas);
void ora_corrupt(uint64_t seed, int step, int B, int N, int V, const float* rate,
                 const int32_t* clean, int32_t* out);
float ora_xent(const float* logits, int rows, int V, const int32_t* target, float* loss);

static uint64_t state = 88172645463325252ull;
static float uniform(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (float)((state >> 40) + 0.5) / 16777216.0f;
}

int main(void) {
    const int Vs[] = {1, 8, 63, 1001, 65536 + 17};
    for (int vi = 0; vi < 5; ++vi) {
        const int B = 3, N = 17, V = Vs[vi];
        float* logits = malloc(sizeof(float) * B * N * V);
        for (long k = 0; k < (long)B * N * V; ++k) logits[k] = 6.0f * (uniform() - 0.5f);
        if (V > 8) {
            logits[(long)1 * N * V + 3] = NAN;
            logits[(long)2 * N * V + 5 * V + 7] = INFINITY;
        }
        int32_t* canvas = malloc(sizeof(int32_t) * B * N);
        int32_t* argmax = calloc(B * N, sizeof(int32_t));
        uint8_t* lock = calloc(B * N, 1);
        float* stats = calloc(B * N * 4, sizeof(float));
        int32_t stop[3] = {0, 0, 0};
        ora_canvas_init(5, vi, B, N, V, canvas);
        for (int step = 0; step < 3; ++step) {
            ora_sample_update(step & 1, 0.1f, 0.8f, 0.4f, 0.005f, 1, 3, 11, step, B, N, V,
                              logits, canvas, argmax, lock, stats, stop);
        }
        stop[0] = stop[1] = stop[2] = 0;
        for (int K = 1; K <= 64; K *= 8)
            ora_sample_update_topk(1, 0.1f, 0.8f, 0.4f, 0.005f, 0, 5, 13, 1, K, B, N, V, logits,
                                   canvas, argmax, lock, stats, stop);
        float rate[3] = {0.0f, 0.5f, 1.0f};
        int32_t* out = malloc(sizeof(int32_t) * B * N);
        ora_corrupt(17, 2, B, N, V, rate, canvas, out);
        float* loss = malloc(sizeof(float) * B * N);
        (void)ora_xent(logits, B * N, V, out, loss);
        free(logits); free(canvas); free(argmax); free(lock); free(stats); free(out); free(loss);
    }
    printf("sampler checks ok\n");
    return 0;
}
