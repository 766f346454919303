/*
 * oracle/sampler.c -- CPU oracle of the multinomial-diffusion sampler.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only tests/, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code with the HIP library.
 *
 * What the pages fix (report-summary page on DiffusionGemma, animattoys.com):
 *   - section 1: the canvas starts as uniformly random vocabulary tokens and
 *     uncertain positions are replaced by *any* vocabulary token (multinomial,
 *     not masked, diffusion); locked tokens may still change later;
 *   - section 4: positions are ordered by entropy, locked from the most
 *     certain one while the running entropy total stays within 0.1, the rest
 *     are re-randomised; temperature starts at 0.8 and falls linearly to 0.4;
 *     generation stops early once the mean entropy is below 0.005 and the
 *     most likely sequence is unchanged between two rounds, with a budget of
 *     48 rounds.
 * The pages say nothing about floating-point arithmetic.  Decisions (the drawn
 * token, lock set, stop flag) are integer outcomes of float computations, so
 * this file fixes the arithmetic completely -- every operation is an IEEE
 * binary32 operation in the order written here, with fma only where written --
 * and the GPU sampler implements the same definition independently.  The
 * definition (chunk layout, merge rule, three-level draw) is this library's
 * own reading of the pages, written out in the functions below.
 *
 * Build: gcc -O2 -std=gnu11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (contraction off: a*b+c must stay two roundings unless fmaf is written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* binary32 helpers                                                    */
/* ------------------------------------------------------------------ */
static float bits_to_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/*
 * ora_exp(x) = e^x for x <= 0, Cody & Waite range reduction.
 *   k = rint(x * log2(e)),  r = x - k*ln2 (two-part ln2, each step one fma),
 *   e^r by its Taylor series to degree 6 in Horner form (one fma per step),
 *   result = p * 2^k with 2^k built from exponent bits.
 * x < -87 (and -inf, NaN) gives +0, so no subnormal is ever produced:
 * for x >= -87 the smallest k is -126 and then r > 0.33, so p*2^k is normal.
 * e^0 = 1 exactly.
 */
float ora_exp(float x)
{
    if (!(x >= -87.0f)) return 0.0f;
    const float LOG2E  = 1.44269504088896341f;
    const float LN2_HI = 0.693145751953125f;       /* 0x3F317200, 9 low bits clear */
    const float LN2_LO = 1.42860682030941723e-06f; /* ln2 - LN2_HI                  */
    float kf = rintf(x * LOG2E);
    float r = fmaf(-kf, LN2_HI, x);
    r = fmaf(-kf, LN2_LO, r);
    float p = 1.0f / 720.0f;
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int k = (int)kf;
    float scale = bits_to_f((uint32_t)(k + 127) << 23);
    return p * scale;
}

/*
 * ora_log(x) = ln x for finite x >= 1 (the sampler only takes logs of
 * softmax normalisers, which are >= 1).  x = 2^e * m with m in (sqrt(1/2),
 * sqrt(2)], f = (m-1)/(m+1), ln m = 2 atanh f = 2f (1 + f^2/3 + ... + f^12/13),
 * ln x = e*ln2 + ln m with ln2 split in two parts.
 */
float ora_log(float x)
{
    const float LN2_HI = 0.693145751953125f;
    const float LN2_LO = 1.42860682030941723e-06f;
    uint32_t b = f_to_bits(x);
    int e = (int)((b >> 23) & 0xffu) - 127;
    float m = bits_to_f((b & 0x7fffffu) | 0x3f800000u);
    if (m > 1.41421356f) { m = m * 0.5f; e = e + 1; }
    float f = (m - 1.0f) / (m + 1.0f);
    float f2 = f * f;
    float q = 1.0f / 13.0f;
    q = fmaf(q, f2, 1.0f / 11.0f);
    q = fmaf(q, f2, 1.0f / 9.0f);
    q = fmaf(q, f2, 1.0f / 7.0f);
    q = fmaf(q, f2, 1.0f / 5.0f);
    q = fmaf(q, f2, 1.0f / 3.0f);
    q = fmaf(q, f2, 1.0f);
    float lm = (2.0f * f) * q;
    float ef = (float)e;
    return fmaf(ef, LN2_HI, fmaf(ef, LN2_LO, lm));
}

/* ------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: */
/* as easy as 1, 2, 3", SC'11).                                        */
/* ------------------------------------------------------------------ */
static uint64_t mulhi64(uint64_t a, uint64_t b)
{
    return (uint64_t)(((unsigned __int128)a * (unsigned __int128)b) >> 64);
}

void ora_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t hi0 = mulhi64(M0, c0), lo0 = M0 * c0;
        uint64_t hi1 = mulhi64(M1, c2), lo1 = M1 * c2;
        uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* A uniform in (0,1) from the top 23 bits of a 64-bit word: (2r+1) / 2^24. */
float ora_uniform(uint64_t o)
{
    uint32_t r = (uint32_t)(o >> 41);
    return (float)(2u * r + 1u) * 5.9604644775390625e-08f; /* 2^-24 */
}

/* A uniform token in [0, V): the high word of o * V. */
int32_t ora_uniform_token(uint64_t o, int32_t V)
{
    return (int32_t)mulhi64(o, (uint64_t)(uint32_t)V);
}

/* The four 64-bit words for (key = seed, counter = (a, b, c, stream)). */
static void draw_block(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t stream,
                       uint64_t out[4])
{
    uint64_t ctr[4] = {a, b, c, stream};
    uint64_t key[2] = {seed, 0};
    ora_philox4x64(ctr, key, out);
}

/* ------------------------------------------------------------------ */
/* Chunk layout of one logit row (a fixed partition of [0, V)).        */
/*   A "tile" is 65536 consecutive entries viewed as 16 x 1024 groups  */
/*   of 4.  Chunk c = t*1024 + lam holds, for d = 0..15 and q = 0..3,  */
/*   entry k = 4*(t*16384 + d*1024 + lam) + q, if k < V, in that order */
/*   (which is increasing k).  A superchunk is 64 consecutive chunks.  */
/* ------------------------------------------------------------------ */
enum { NLANE = 1024, NDEPTH = 16, TILE = 4 * NLANE * NDEPTH, SUPER = 64 };

static int chunk_member(int V, int c, int idx /* 0..63 */)
{
    int t = c / NLANE, lam = c % NLANE;
    int d = idx / 4, q = idx % 4;
    long k = 4L * ((long)t * NLANE * NDEPTH + (long)d * NLANE + lam) + q;
    return k < V ? (int)k : -1;
}

typedef struct { float m; int32_t j; float s; float a; float s2; } chunk_t;

/* Stats of one chunk: max, first argmax, and sequential sums of
 * e = E(z), e*z and w = E(z*invT) with z = l - max. s == 0 marks empty; a
 * NaN s marks a chunk whose maximum is not finite. */
static chunk_t chunk_stats(const float* row, int V, int c, float invT)
{
    chunk_t r = {-INFINITY, -1, 0.0f, 0.0f, 0.0f};
    for (int idx = 0; idx < 4 * NDEPTH; ++idx) {
        int k = chunk_member(V, c, idx);
        if (k < 0) continue;
        if (row[k] > r.m || r.j < 0) { r.m = row[k]; r.j = k; }
    }
    if (r.j < 0) return r;
    for (int idx = 0; idx < 4 * NDEPTH; ++idx) {
        int k = chunk_member(V, c, idx);
        if (k < 0) continue;
        float z = row[k] - r.m;
        float e = ora_exp(z);
        r.s = r.s + e;
        r.a = r.a + e * z;
        r.s2 = r.s2 + ora_exp(z * invT);
    }
    /* a chunk whose maximum is not finite (a NaN first member, or an
     * infinite logit) is marked by a NaN sum, so that its row's entropy is
     * NaN: every non-finite logit shows (see ora_nonfinite) */
    if (!(r.m - r.m == 0.0f)) r.s = NAN;
    return r;
}

/* Merge of two (m, j, s, a) summaries; symmetric bit for bit. */
static chunk_t merge(chunk_t x, chunk_t y)
{
    if (x.s == 0.0f) return y;
    if (y.s == 0.0f) return x;
    chunk_t r;
    r.m = x.m > y.m ? x.m : y.m;
    r.j = x.m > y.m ? x.j : (y.m > x.m ? y.j : (x.j < y.j ? x.j : y.j));
    float dx = x.m - r.m, dy = y.m - r.m;
    float fx = ora_exp(dx), fy = ora_exp(dy);
    r.s = x.s * fx + y.s * fy;
    r.a = fx * (x.a + dx * x.s) + fy * (y.a + dy * y.s);
    r.s2 = 0.0f;
    return r;
}

/* Halves-recursion tree over v[lo, lo+n), n a power of two. */
static chunk_t tree(const chunk_t* v, int lo, int n)
{
    if (n == 1) return v[lo];
    return merge(tree(v, lo, n / 2), tree(v, lo + n / 2, n / 2));
}

static int n_tiles(int V) { return (V + TILE - 1) / TILE; }

/* Row summary and per-chunk records.  chunks must hold n_tiles(V)*1024. */
static chunk_t row_stats(const float* row, int V, float invT, chunk_t* chunks)
{
    int nt = n_tiles(V);
    for (int c = 0; c < nt * NLANE; ++c) chunks[c] = chunk_stats(row, V, c, invT);
    chunk_t* fold = (chunk_t*)malloc(sizeof(chunk_t) * NLANE);
    for (int lam = 0; lam < NLANE; ++lam) {
        chunk_t f = chunks[lam];
        for (int t = 1; t < nt; ++t) f = merge(f, chunks[t * NLANE + lam]);
        fold[lam] = f;
    }
    chunk_t r = tree(fold, 0, NLANE);
    free(fold);
    return r;
}

/* Entropy (nats) and max-probability of the T = 1 distribution. */
static void entropy_maxprob(chunk_t r, float* H, float* pmax)
{
    float h = ora_log(r.s) - r.a / r.s;
    *H = h > 0.0f ? h : (h != h ? h : 0.0f);   /* a NaN (non-finite logits) stays NaN */
    *pmax = 1.0f / r.s;
}

/* Inverse-CDF pick over w[0..n): first i with running sum > u * total,
 * else the last i with w > 0. */
static int pick(const float* w, int n, float u)
{
    float total = 0.0f;
    for (int i = 0; i < n; ++i) total = total + w[i];
    float target = u * total;
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) {
        acc = acc + w[i];
        if (acc > target) return i;
    }
    for (int i = n - 1; i >= 0; --i)
        if (w[i] > 0.0f) return i;
    return 0;
}

/* Draw from softmax(row / T): superchunk, then chunk, then entry. */
static int32_t draw_token(const float* row, int V, float invT, const chunk_t* chunks,
                          float m, float u1, float u2, float u3)
{
    int nt = n_tiles(V);
    int nchunk = nt * NLANE, nsuper = nchunk / SUPER;
    float* G = (float*)malloc(sizeof(float) * nchunk);
    for (int c = 0; c < nchunk; ++c)
        G[c] = chunks[c].s == 0.0f ? 0.0f : chunks[c].s2 * ora_exp((chunks[c].m - m) * invT);
    float* W = (float*)malloc(sizeof(float) * nsuper);
    for (int sc = 0; sc < nsuper; ++sc) {
        float acc = 0.0f;
        for (int i = 0; i < SUPER; ++i) acc = acc + G[sc * SUPER + i];
        W[sc] = acc;
    }
    int sstar = pick(W, nsuper, u1);
    int cstar = sstar * SUPER + pick(G + sstar * SUPER, SUPER, u2);
    float w[4 * NDEPTH];
    int kk[4 * NDEPTH];
    int n = 0;
    for (int idx = 0; idx < 4 * NDEPTH; ++idx) {
        int k = chunk_member(V, cstar, idx);
        if (k < 0) continue;
        w[n] = ora_exp((row[k] - chunks[cstar].m) * invT);
        kk[n] = k;
        ++n;
    }
    int32_t y = n > 0 ? kk[pick(w, n, u3)] : 0;
    free(G);
    free(W);
    return y;
}

/* ------------------------------------------------------------------ */
/* Public oracle entry points (called from Python through ctypes).     */
/* ------------------------------------------------------------------ */

/* Per-row statistics: out4 = {max logit, S = sum exp(l - max), H, pmax},
 * argmax (first index of the maximum). */
void ora_row_stats(const float* row, int V, float* out4, int32_t* argmax)
{
    chunk_t* chunks = (chunk_t*)malloc(sizeof(chunk_t) * n_tiles(V) * NLANE);
    chunk_t r = row_stats(row, V, 1.0f, chunks);
    float H, p;
    entropy_maxprob(r, &H, &p);
    out4[0] = r.m; out4[1] = r.s; out4[2] = H; out4[3] = p;
    *argmax = r.j;
    free(chunks);
}

/* One categorical draw from softmax(row * invT) with explicit uniforms. */
int32_t ora_draw(const float* row, int V, float invT, float u1, float u2, float u3)
{
    chunk_t* chunks = (chunk_t*)malloc(sizeof(chunk_t) * n_tiles(V) * NLANE);
    chunk_t r = row_stats(row, V, invT, chunks);
    int32_t y = draw_token(row, V, invT, chunks, r.m, u1, u2, u3);
    free(chunks);
    return y;
}

/* Temperature of step t: T0 + (T1 - T0) * t / (max_steps - 1), in double,
 * rounded to binary32; returns 1/T in binary32. */
float ora_inv_temperature(float T0, float T1, int t, int max_steps)
{
    double T = (double)T0;
    if (max_steps > 1) T = (double)T0 + ((double)T1 - (double)T0) * (double)t / (double)(max_steps - 1);
    float Tf = (float)T;
    return 1.0f / Tf;
}

/* Canvas initialisation for block `block`: N uniform tokens per canvas,
 * Philox counter (block, b, i, 1), first output word. */
void ora_canvas_init(uint64_t seed, int block, int B, int N, int V, int32_t* canvas)
{
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i) {
            uint64_t o[4];
            draw_block(seed, (uint64_t)block, (uint64_t)b, (uint64_t)i, 1, o);
            canvas[b * N + i] = ora_uniform_token(o[0], V);
        }
}

/* ------------------------------------------------------------------ */
/* Training-side forward (report-summary page, section 1: training     */
/* replaces a random share of a sentence's tokens, from 0 % to 100 %,  */
/* by junk and asks for the original; section 3: the supervised stage  */
/* does this at varying degrees and trains on the gap between the       */
/* prediction and the original).  Plainest reading, written out:        */
/*   corruption: position (b, i) of canvas b with rate r_b draws the    */
/*     Philox block of counter (step, b, i, 2), key (seed, 0); it is    */
/*     replaced iff uniform(word 0) < r_b, by uniform_token(word 1, V)  */
/*     (the multinomial kind of section 1: any token, possibly the      */
/*     original one);                                                   */
/*   loss of a position: the cross-entropy of softmax(l) at the clean  */
/*     token x, -ln p(x) = ln S - (l[x] - m), with m and S the row's    */
/*     max and sum of E(l - m) as the sampler defines them, so         */
/*     loss = L(S) - (l[x] - m) in binary32 (both steps as written);    */
/*   mean loss: the sequential binary32 sum over positions in order,    */
/*     divided by their count (converted to binary32).                  */
/* ------------------------------------------------------------------ */

void ora_corrupt(uint64_t seed, int step, int B, int N, int V, const float* rate,
                 const int32_t* clean, int32_t* out)
{
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i) {
            uint64_t o[4];
            draw_block(seed, (uint64_t)step, (uint64_t)b, (uint64_t)i, 2, o);
            size_t bi = (size_t)b * N + i;
            out[bi] = ora_uniform(o[0]) < rate[b] ? ora_uniform_token(o[1], V) : clean[bi];
        }
}

/* Cross-entropy of each row [rows][V] at target[r]; returns the mean. */
float ora_xent(const float* logits, int rows, int V, const int32_t* target, float* loss)
{
    chunk_t* chunks = (chunk_t*)malloc(sizeof(chunk_t) * n_tiles(V) * NLANE);
    float sum = 0.0f;
    for (int r = 0; r < rows; ++r) {
        const float* row = logits + (size_t)r * V;
        chunk_t st = row_stats(row, V, 1.0f, chunks);
        float z = row[target[r]] - st.m;
        loss[r] = ora_log(st.s) - z;
        sum = sum + loss[r];
    }
    free(chunks);
    return sum / (float)rows;
}

/* Lock set of one canvas from per-position entropy H and max-probability P.
 * rule 0 (max-probability): lock i  <=>  P[i] > theta.
 * rule 1 (cumulative entropy, report-summary page section 4): visit positions
 * by (H, index) ascending, lock while the running entropy total plus the
 * next H stays <= theta; the first position that would exceed it, and all
 * after it, stay unlocked. */
void ora_lock_set(int rule, float theta, int N, const float* H, const float* P, uint8_t* lock)
{
    if (rule == 0) {
        for (int i = 0; i < N; ++i) lock[i] = P[i] > theta ? 1 : 0;
        return;
    }
    int* order = (int*)malloc(sizeof(int) * (N > 0 ? N : 1));
    for (int i = 0; i < N; ++i) { order[i] = i; lock[i] = 0; }
    for (int i = 1; i < N; ++i) { /* insertion sort by (H, index) */
        int v = order[i], j = i - 1;
        while (j >= 0 && (H[order[j]] > H[v] || (H[order[j]] == H[v] && order[j] > v))) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = v;
    }
    float acc = 0.0f;
    for (int n = 0; n < N; ++n) {
        int i = order[n];
        if (acc + H[i] <= theta) { lock[i] = 1; acc = acc + H[i]; }
        else break;
    }
    free(order);
}

/* Non-finite logits.  Under the arithmetic above a NaN or infinite logit
 * makes its row's sum of e*z NaN (0 * inf or NaN), hence its entropy NaN;
 * the pages assume finite scores.  Reading: such a canvas is reported
 * (stop = 2) and left as it was (canvas, argmax and locks untouched), so a
 * caller can tell a numerical failure from a stop. */
int ora_nonfinite(int N, const float* H)
{
    for (int i = 0; i < N; ++i)
        if (H[i] != H[i]) return 1;
    return 0;
}

/* Stop flag of one canvas (report-summary page section 4): mean entropy
 * (sequential binary32 sum in position order, divided by N) below tau and,
 * if required, the most likely sequence unchanged from the previous round;
 * or the round budget is used up. */
int ora_stop_flag(int N, const float* H, int stable, float tau, int require_stable, int step,
                  int max_steps)
{
    float sumH = 0.0f;
    for (int i = 0; i < N; ++i) sumH = sumH + H[i];
    float meanH = sumH / (float)N;
    int st = (meanH < tau) && (!require_stable || stable);
    if (step + 1 >= max_steps) st = 1;
    return st;
}

/* ------------------------------------------------------------------ */
/* Top-k truncation (report-summary page, section 9, known limitations:  */
/* top-k truncation of the distribution is the named missing            */
/* throughput optimisation).  With K > 0 a position's statistics, draw  */
/* and self-conditioning use only its K largest logits.                 */
/*   candidates c_0..c_{K-1}: the K largest entries, ordered by value    */
/*     descending, ties to the lower index (a total order); a NaN ranks */
/*     above every number, NaNs tie among themselves (reading: the pages */
/*     assume finite scores; this order, that of a positive NaN in IEEE  */
/*     754 totalOrder, puts any NaN or +inf among the candidates, so the */
/*     row's statistics turn NaN and its canvas is reported);           */
/*   m = l[c_0] (the argmax); z_i = l[c_i] - m; e_i = ora_exp(z_i);      */
/*   S = e_0 + e_1 + ... (in candidate order), A likewise of e_i * z_i;  */
/*   H = max(0, ora_log(S) - A / S), pmax = 1 / S;                       */
/*   draw: w_i = ora_exp(z_i * invT), y = c_pick(w, K, u) with u from    */
/*     Philox word 0 (one level; words 2 and 3 are not used);           */
/*   self-conditioning weights p_i = e_i / S.                            */
/* ------------------------------------------------------------------ */
static const float* g_row;   /* qsort has no context argument */
static int cmp_desc(const void* pa, const void* pb)
{
    int a = *(const int*)pa, b = *(const int*)pb;
    float x = g_row[a], y = g_row[b];
    int xn = x != x, yn = y != y;
    if (xn != yn) return xn ? -1 : 1;
    if (x > y) return -1;
    if (x < y) return 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* One row: out4 = {m, S, H, pmax}; idx[K], p[K] the candidates and their
 * self-conditioning weights; returns the drawn token. */
int32_t ora_topk_row(const float* row, int V, int K, float invT, float u, float* out4,
                     int32_t* idx, float* p)
{
    int* ord = (int*)malloc(sizeof(int) * V);
    for (int v = 0; v < V; ++v) ord[v] = v;
    g_row = row;
    qsort(ord, V, sizeof(int), cmp_desc);
    if (K > V) K = V;
    float m = row[ord[0]];
    float S = 0.0f, A = 0.0f;
    float* e = (float*)malloc(sizeof(float) * K);
    float* w = (float*)malloc(sizeof(float) * K);
    for (int i = 0; i < K; ++i) {
        float z = row[ord[i]] - m;
        e[i] = ora_exp(z);
        S = S + e[i];
        float ez = e[i] * z;
        A = A + ez;
        w[i] = ora_exp(z * invT);
    }
    float h = ora_log(S) - A / S;
    out4[0] = m;
    out4[1] = S;
    out4[2] = h > 0.0f ? h : (h != h ? h : 0.0f);
    out4[3] = 1.0f / S;
    for (int i = 0; i < K; ++i) {
        idx[i] = ord[i];
        p[i] = e[i] / S;
    }
    int32_t y = ord[pick(w, K, u)];
    free(ord); free(e); free(w);
    return y;
}

/* ora_sample_update with top-k truncation (K >= 1); argmax = c_0. */
void ora_sample_update_topk(int lock_rule, float theta, float T0, float T1, float tau,
                            int require_stable, int max_steps, uint64_t seed, int step, int K,
                            int B, int N, int V, const float* logits, int32_t* canvas,
                            int32_t* argmax, uint8_t* lock, float* stats, int32_t* stop)
{
    float invT = ora_inv_temperature(T0, T1, step, max_steps);
    float* H = (float*)malloc(sizeof(float) * N);
    float* P = (float*)malloc(sizeof(float) * N);
    int32_t* y = (int32_t*)malloc(sizeof(int32_t) * N);
    int32_t* r = (int32_t*)malloc(sizeof(int32_t) * N);
    int32_t* am = (int32_t*)malloc(sizeof(int32_t) * N);
    int Ke = K < V ? K : V;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * Ke);
    float* pp = (float*)malloc(sizeof(float) * Ke);
    for (int b = 0; b < B; ++b) {
        if (stop[b]) continue;
        for (int i = 0; i < N; ++i) {
            const float* row = logits + ((size_t)b * N + i) * (size_t)V;
            uint64_t o[4];
            draw_block(seed, (uint64_t)step, (uint64_t)b, (uint64_t)i, 0, o);
            float* st = stats + ((size_t)b * N + i) * 4;
            y[i] = ora_topk_row(row, V, K, invT, ora_uniform(o[0]), st, idx, pp);
            H[i] = st[2];
            P[i] = st[3];
            am[i] = idx[0];
            r[i] = ora_uniform_token(o[1], V);
        }
        if (ora_nonfinite(N, H)) { stop[b] = 2; continue; }
        ora_lock_set(lock_rule, theta, N, H, P, lock + (size_t)b * N);
        uint8_t* lk = lock + (size_t)b * N;
        int stable = step > 0;
        for (int i = 0; i < N; ++i) {
            size_t bi = (size_t)b * N + i;
            canvas[bi] = lk[i] ? y[i] : r[i];
            if (argmax[bi] != am[i]) stable = 0;
            argmax[bi] = am[i];
        }
        stop[b] = ora_stop_flag(N, H, stable, tau, require_stable, step, max_steps);
    }
    free(H); free(P); free(y); free(r); free(am); free(idx); free(pp);
}

/*
 * One sampler update over B canvases of N positions each.
 *   logits   [B,N,V] float
 *   canvas   [B,N] in/out   argmax [B,N] in: previous step, out: this step
 *   lock     [B,N] out      stats [B,N,4] out {m, S, H, pmax}
 *   stop     [B] in/out: canvases with stop != 0 are left untouched; a canvas
 *            whose logits are not all finite gets stop = 2 and keeps its
 *            canvas, argmax and locks (its statistics are written).
 * lock_rule 0 = max-probability (pmax > theta), 1 = cumulative entropy.
 */
void ora_sample_update(int lock_rule, float theta, float T0, float T1, float tau,
                       int require_stable, int max_steps, uint64_t seed, int step,
                       int B, int N, int V, const float* logits, int32_t* canvas,
                       int32_t* argmax, uint8_t* lock, float* stats, int32_t* stop)
{
    float invT = ora_inv_temperature(T0, T1, step, max_steps);
    chunk_t* chunks = (chunk_t*)malloc(sizeof(chunk_t) * n_tiles(V) * NLANE);
    float* H = (float*)malloc(sizeof(float) * N);
    float* P = (float*)malloc(sizeof(float) * N);
    int32_t* y = (int32_t*)malloc(sizeof(int32_t) * N);
    int32_t* r = (int32_t*)malloc(sizeof(int32_t) * N);
    int32_t* am = (int32_t*)malloc(sizeof(int32_t) * N);
    for (int b = 0; b < B; ++b) {
        if (stop[b]) continue;
        for (int i = 0; i < N; ++i) {
            const float* row = logits + ((size_t)b * N + i) * (size_t)V;
            chunk_t s = row_stats(row, V, invT, chunks);
            entropy_maxprob(s, &H[i], &P[i]);
            am[i] = s.j;
            uint64_t o[4];
            draw_block(seed, (uint64_t)step, (uint64_t)b, (uint64_t)i, 0, o);
            y[i] = draw_token(row, V, invT, chunks, s.m, ora_uniform(o[0]), ora_uniform(o[2]),
                              ora_uniform(o[3]));
            r[i] = ora_uniform_token(o[1], V);
            float* st = stats + ((size_t)b * N + i) * 4;
            st[0] = s.m; st[1] = s.s; st[2] = H[i]; st[3] = P[i];
        }
        if (ora_nonfinite(N, H)) { stop[b] = 2; continue; }
        ora_lock_set(lock_rule, theta, N, H, P, lock + (size_t)b * N);
        uint8_t* lk = lock + (size_t)b * N;
        /* renoise and stop */
        int stable = step > 0;
        for (int i = 0; i < N; ++i) {
            size_t bi = (size_t)b * N + i;
            canvas[bi] = lk[i] ? y[i] : r[i];
            if (argmax[bi] != am[i]) stable = 0;
            argmax[bi] = am[i];
        }
        stop[b] = ora_stop_flag(N, H, stable, tau, require_stable, step, max_steps);
    }
    free(chunks); free(H); free(P); free(y); free(r); free(am);
}
