/*
 * Seeded synthetic input generator shared by the tests, the bench and the
 * smoke check.  It holds no attention arithmetic: it only turns
 * (seed, tensor id, element index) into a bf16 bit pattern.
 *
 * Definition (counter based, so any element can be produced on its own and
 * any thread split gives the same bits):
 *   key      = splitmix64(seed) ^ splitmix64(tensor_id + 0x5EED)
 *   stream_n = splitmix64(key + n * GAMMA)      (SplitMix64, Steele/Lea/Flood 2014)
 *   element i draws stream_{2i} and stream_{2i+1}:
 *     u1 = ((s0 >> 11) + 1) * 2^-53  in (0, 1]
 *     u2 =  (s1 >> 11)      * 2^-53  in [0, 1)
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller)
 *   bf16 = round-to-nearest-even(float(z))
 *
 * Outlier channels: kbg_outlier_channels picks n distinct channel indices in
 * [0, head_dim) from the seed; kbg_scale_channels multiplies those channels of
 * every row by 2^k (exact in bf16 for normal values).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t splitmix64(uint64_t x) {
    x += GAMMA;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
    return splitmix64(seed) ^ splitmix64(tensor_id + 0x5EEDull);
}

uint16_t kbg_normal_bf16_at(uint64_t seed, uint64_t tensor_id, uint64_t i) {
    const uint64_t key = stream_key(seed, tensor_id);
    const uint64_t s0 = splitmix64(key + (2 * i) * GAMMA);
    const uint64_t s1 = splitmix64(key + (2 * i + 1) * GAMMA);
    const double u1 = (double)((s0 >> 11) + 1) * 0x1.0p-53;
    const double u2 = (double)(s1 >> 11) * 0x1.0p-53;
    const double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
    return f32_to_bf16_rne((float)z);
}

typedef struct {
    uint64_t seed, tensor_id, begin, end;
    uint16_t* out;
} job_t;

static void* normal_worker(void* arg) {
    job_t* j = (job_t*)arg;
    for (uint64_t i = j->begin; i < j->end; ++i) j->out[i] = kbg_normal_bf16_at(j->seed, j->tensor_id, i);
    return NULL;
}

/* Fill out[0..n) with element indices [0, n) of the tensor's stream. */
int kbg_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t n, uint16_t* out, int threads) {
    if (!out && n) return -1;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((uint64_t)threads > n / 4096 + 1) threads = (int)(n / 4096 + 1);
    pthread_t tid[256];
    job_t jobs[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t].seed = seed;
        jobs[t].tensor_id = tensor_id;
        jobs[t].begin = n * (uint64_t)t / (uint64_t)threads;
        jobs[t].end = n * (uint64_t)(t + 1) / (uint64_t)threads;
        jobs[t].out = out;
    }
    for (int t = 1; t < threads; ++t)
        if (pthread_create(&tid[t], NULL, normal_worker, &jobs[t]) != 0) return -2;
    normal_worker(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
    return 0;
}

/* n distinct channel indices in [0, head_dim), drawn from the seed. */
int kbg_outlier_channels(uint64_t seed, int n, int head_dim, int32_t* out) {
    if (n < 0 || n > head_dim || !out) return -1;
    uint64_t key = stream_key(seed, 0x0C7A11E5ull);
    int found = 0;
    for (uint64_t c = 0; found < n; ++c) {
        int ch = (int)(splitmix64(key + c * GAMMA) % (uint64_t)head_dim);
        int dup = 0;
        for (int i = 0; i < found; ++i) dup |= (out[i] == ch);
        if (!dup) out[found++] = ch;
    }
    return 0;
}

/* x viewed as [rows, head_dim]: multiply the listed channels by 2^log2_factor. */
int kbg_scale_channels(uint16_t* x, uint64_t rows, int head_dim, const int32_t* ch, int n, int log2_factor) {
    if (!x || !ch || head_dim <= 0) return -1;
    const float f = ldexpf(1.0f, log2_factor);
    for (uint64_t r = 0; r < rows; ++r)
        for (int i = 0; i < n; ++i) {
            uint16_t* e = x + r * (uint64_t)head_dim + (uint64_t)ch[i];
            *e = f32_to_bf16_rne(bf16_to_f32(*e) * f);
        }
    return 0;
}
