/*
 * moeq_synth.h - seeded synthetic input fill on the GPU.
 *
 * Input generation only: it writes bytes drawn from a counter-based generator
 * and maps them onto the code ranges a workload uses; it decodes nothing. The
 * host generator in bit_quantized_moe_dequant_amd/synth.py implements the same
 * definition, so any range of a device-filled tensor can be regenerated on the
 * host:
 *
 *   mix64(z)      = SplitMix64 finaliser (Steele, Lea, Flood, OOPSLA 2014;
 *                   constants 0xBF58476D1CE4E5B9, 0x94D049BB133111EB)
 *   key(S, s)     = mix64(S << 32 | s)        (S, s taken mod 2^32)
 *   word(S, s, i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   byte j of stream s = byte (j % 8), little-endian, of word(S, s, j / 8)
 */
#ifndef MOEQ_SYNTH_H_
#define MOEQ_SYNTH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEQ_FIELD_RAW 0          /* bytes as drawn */
#define MOEQ_FIELD_E8M0_119_123 1 /* 119 + b % 5 */
#define MOEQ_FIELD_E4M3_08_28 2   /* 0x08 + b % 33 */
#define MOEQ_FIELD_E4M3_FINITE 3  /* c = b % 254, c + 1 if c >= 0x7f */
#define MOEQ_FIELD_Q2K_BLOCK 4    /* 84-byte blocks; fp16 at offsets 80 and 82 = d_table[u16 % 4096] */
#define MOEQ_FIELD_IQ2_BLOCK 5    /* 66-byte blocks; fp16 at offset 0 = d_table[u16 % 4096] */

/* Write bytes [byte_offset, byte_offset + nbytes) of stream `stream` under seed
 * `seed`, mapped by `field`, to dst (device). d_table: device u16[4096] for the
 * block fields (else may be NULL). Block fields need byte_offset and nbytes to be
 * whole blocks. Returns 0 or a negative moeq status. */
int moeq_synth_fill(uint8_t* dst, size_t nbytes, uint64_t seed, uint32_t stream, uint64_t byte_offset, int field,
                    const uint16_t* d_table, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_SYNTH_H_ */
