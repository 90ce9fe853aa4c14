/*
 * Seeded synthetic expert-weight generator, host side.
 *
 * Input generation only: nothing in this file is part of the MoE arithmetic.
 * The device twin (gen_device.hip) implements the same counter-based stream
 * so that a byte generated on the GPU equals the byte generated here.
 *
 * Stream definition (SplitMix64, Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014, with the finaliser constants
 * of Vigna's splitmix64.c): the i-th output (i >= 0) of a SplitMix64 seeded
 * with state s is mix(s + (i + 1) * GAMMA).  Because that is a closed form in
 * i, any byte can be generated independently of every other.
 *
 *   stream(seed, layer, expert, tensor) = out_{(layer<<32)|(expert<<8)|tensor}(seed)
 *   nibble byte o of a stream  = byte (o & 7) of out_{o>>3}(stream)   (little end)
 *   scale  byte o of a stream  = lo + ((out_o(stream) >> 32) * (hi-lo+1)) >> 32
 *
 * Tensor ids: 0 w1, 1 s1, 2 w3, 3 s3, 4 w2, 5 s2.
 */
#include <stdint.h>
#include <stddef.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_sm64_at(uint64_t state, uint64_t i) {
    return sm64_mix(state + (i + 1) * SM64_GAMMA);
}

uint64_t synth_stream(uint64_t seed, uint32_t layer, uint32_t expert, uint32_t tensor) {
    uint64_t ctr = ((uint64_t)layer << 32) | ((uint64_t)expert << 8) | (uint64_t)(tensor & 0xFF);
    return synth_sm64_at(seed, ctr);
}

/* Fill dst[0..n) with bytes [off, off+n) of stream `st`.
 * kind 0: uniform bytes (two uniform E2M1 nibbles each); kind 1: scale bytes in [lo, hi]. */
void synth_fill(uint8_t *dst, int64_t off, int64_t n, uint64_t st, int kind, int lo, int hi) {
    if (kind == 0) {
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            int64_t o = off + i;
            uint64_t h = synth_sm64_at(st, (uint64_t)(o >> 3));
            dst[i] = (uint8_t)(h >> (8 * (o & 7)));
        }
    } else {
        uint64_t span = (uint64_t)(hi - lo + 1);
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            uint64_t h = synth_sm64_at(st, (uint64_t)(off + i));
            dst[i] = (uint8_t)(lo + (int)(((h >> 32) * span) >> 32));
        }
    }
}
