/* Host implementation of the counter-based Q8_0 block generator described in
 * workloads/__init__.py (SplitMix64 outputs; 17 outputs per 34-byte block).
 * Input generation only: no part of the quantised FFN is computed here. */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Blocks [first, first + n) of stream `key` into dst (n * 34 bytes). */
void synth_q8_0_blocks(uint64_t key, int64_t first, int64_t n, uint8_t* dst) {
    for (int64_t i = 0; i < n; ++i) {
        const uint64_t b = (uint64_t)(first + i);
        int8_t q[32];
        for (int t = 0; t < 16; ++t) {
            const uint64_t o = mix64(key + (b * 17 + (uint64_t)t + 1) * GAMMA);
            for (int h = 0; h < 2; ++h) {
                const uint32_t w = (uint32_t)(o >> (32 * h));
                const uint32_t v = (w & 0xFF) + ((w >> 8) & 0xFF) + ((w >> 16) & 0xFF) + (w >> 24);
                int qi = (int)((v * 43u) >> 7) - 171;
                q[2 * t + h] = (int8_t)(qi < -127 ? -127 : (qi > 127 ? 127 : qi));
            }
        }
        const uint64_t o = mix64(key + (b * 17 + 17) * GAMMA);
        q[(o >> 10) & 31] = ((o >> 15) & 1) ? (int8_t)-127 : (int8_t)127;
        const uint16_t d = (uint16_t)(0x0C00u | (uint32_t)(o & 0x3FF));
        uint8_t* p = dst + i * 34;
        p[0] = (uint8_t)(d & 0xFF);
        p[1] = (uint8_t)(d >> 8);
        memcpy(p + 2, q, 32);
    }
}
