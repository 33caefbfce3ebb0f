/*
 * host_floor.c -- the host's streaming-read memory floor, a measurement aid
 * of the benchmark's CPU leg (the oracle timed on the host's cores).
 *
 * TEST AND BENCHMARK INFRASTRUCTURE ONLY, like oracle.c beside it: it holds
 * none of the method's arithmetic, and the product library never links it.
 *
 * bankML "par.rs -- the persistent thread pool and row scheduler", section
 * "How it is verified": the memory floor is a plain streaming read of a
 * buffer far larger than the caches (768 MiB there), at one to several
 * threads; a token's weight stream cannot be read faster than that on the
 * same machine.  Here: every thread reads one contiguous slice of the buffer
 * once per pass with 8-byte loads folded by XOR (so no load can be dropped),
 * and the pass time is the time from the start signal to the last thread's
 * end.
 *
 * Build: gcc -O2 -fPIC -shared host_floor.c -lpthread
 */
#define _POSIX_C_SOURCE 200809L
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

typedef struct {
    const uint64_t *p;
    size_t n; /* words of this thread's slice */
    uint64_t fold;
    atomic_int *go;
} floor_slice;

static double now_s(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static void *read_slice(void *arg)
{
    floor_slice *s = (floor_slice *)arg;
    while (!atomic_load(s->go))
        ;
    uint64_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    size_t i = 0;
    for (; i + 4 <= s->n; i += 4) {
        a0 ^= s->p[i];
        a1 ^= s->p[i + 1];
        a2 ^= s->p[i + 2];
        a3 ^= s->p[i + 3];
    }
    for (; i < s->n; ++i)
        a0 ^= s->p[i];
    s->fold = a0 ^ a1 ^ a2 ^ a3;
    return NULL;
}

/* One pass over buf (words 64-bit words) with `threads` threads; returns the
 * seconds it took and the XOR of all words in *fold. */
static double one_pass(const uint64_t *buf, size_t words, int threads, uint64_t *fold)
{
    floor_slice sl[256];
    pthread_t tid[256];
    atomic_int go;
    atomic_init(&go, 0);
    if (threads > 256)
        threads = 256;
    size_t per = words / (size_t)threads;
    int spawned = 0;
    for (int t = 0; t < threads; ++t) {
        sl[t].p = buf + per * (size_t)t;
        sl[t].n = t == threads - 1 ? words - per * (size_t)t : per;
        sl[t].fold = 0;
        sl[t].go = &go;
        if (t > 0) {
            if (pthread_create(&tid[t], NULL, read_slice, &sl[t]) != 0)
                break;
            ++spawned;
        }
    }
    if (spawned != threads - 1) {
        atomic_store(&go, 1);
        for (int t = 1; t <= spawned; ++t)
            pthread_join(tid[t], NULL);
        return -1.0;
    }
    double t0 = now_s();
    atomic_store(&go, 1);
    read_slice(&sl[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tid[t], NULL);
    double dt = now_s() - t0;
    uint64_t f = 0;
    for (int t = 0; t < threads; ++t)
        f ^= sl[t].fold;
    *fold = f;
    return dt;
}

/* Streaming-read bandwidth in bytes per second of a `bytes` buffer (filled
 * with a known pattern first), for each of the nthreads thread counts in
 * thread_counts: the median of `reps` passes goes to gbs_out[i] (GB/s,
 * 1e9 bytes).  Returns 0, -1 if the buffer cannot be allocated or a thread
 * cannot be started, -2 if a pass read wrong data. */
int host_read_floor(size_t bytes, const int *thread_counts, int nthreads, int reps, double *gbs_out)
{
    size_t words = bytes / 8;
    if (words == 0 || reps < 1 || reps > 64)
        return -1;
    uint64_t *buf = (uint64_t *)aligned_alloc(4096, words * 8);
    if (!buf)
        return -1;
    uint64_t expect = 0;
    for (size_t i = 0; i < words; ++i) {
        buf[i] = (uint64_t)i * 0x9E3779B97F4A7C15ull;
        expect ^= buf[i];
    }
    int rc = 0;
    for (int k = 0; k < nthreads && rc == 0; ++k) {
        double t[64];
        for (int r = 0; r < reps; ++r) {
            uint64_t fold = 0;
            t[r] = one_pass(buf, words, thread_counts[k], &fold);
            if (t[r] <= 0.0) {
                rc = -1;
                break;
            }
            if (fold != expect) {
                rc = -2;
                break;
            }
        }
        if (rc)
            break;
        /* median (insertion sort of at most 64 values) */
        for (int i = 1; i < reps; ++i)
            for (int j = i; j > 0 && t[j] < t[j - 1]; --j) {
                double x = t[j];
                t[j] = t[j - 1];
                t[j - 1] = x;
            }
        double med = reps % 2 ? t[reps / 2] : 0.5 * (t[reps / 2 - 1] + t[reps / 2]);
        gbs_out[k] = (double)(words * 8) / med / 1e9;
    }
    free(buf);
    return rc;
}
