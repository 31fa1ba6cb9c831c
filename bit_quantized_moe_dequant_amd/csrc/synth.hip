// Seeded synthetic input fill (input generation only; see include/moeq_synth.h).
// Implements the SplitMix64 counter-based generator and the field maps that the
// host generator module implements, so device-filled tensors can be regenerated
// on the host for any expert.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"
#include "moeq_synth.h"

namespace {

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ uint32_t raw_byte(uint64_t key, uint64_t pos) {
  uint64_t w = mix64(key + (pos / 8 + 1) * 0x9E3779B97F4A7C15ull);
  return (uint32_t)(w >> (8 * (pos % 8))) & 0xFFu;
}

__device__ __forceinline__ uint32_t map_byte(uint64_t key, uint64_t pos, uint32_t b, int field, const uint16_t* dtab) {
  switch (field) {
    case MOEQ_FIELD_E8M0_119_123: return 119u + b % 5u;
    case MOEQ_FIELD_E4M3_08_28: return 0x08u + b % 33u;
    case MOEQ_FIELD_E4M3_FINITE: {
      uint32_t c = b % 254u;
      return c >= 0x7Fu ? c + 1u : c;
    }
    case MOEQ_FIELD_Q2K_BLOCK:
    case MOEQ_FIELD_IQ2_BLOCK: {
      const uint64_t bs = field == MOEQ_FIELD_Q2K_BLOCK ? 84 : 66;
      const uint64_t r = pos % bs;
      bool lo = field == MOEQ_FIELD_Q2K_BLOCK ? (r == 80 || r == 82) : (r == 0);
      bool hi = field == MOEQ_FIELD_Q2K_BLOCK ? (r == 81 || r == 83) : (r == 1);
      if (lo) {
        uint32_t raw = b | (raw_byte(key, pos + 1) << 8);
        return dtab[raw % 4096u] & 0xFFu;
      }
      if (hi) {
        uint32_t raw = raw_byte(key, pos - 1) | (b << 8);
        return (uint32_t)dtab[raw % 4096u] >> 8;
      }
      return b;
    }
  }
  return b;
}

__global__ __launch_bounds__(256) void k_fill(uint8_t* dst, size_t nbytes, uint64_t key, uint64_t byte_offset,
                                              int field, const uint16_t* dtab) {
  size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= nbytes) return;
  const uint64_t p0 = byte_offset + i;
  if ((byte_offset % 8) == 0 && i + 8 <= nbytes && field != MOEQ_FIELD_Q2K_BLOCK && field != MOEQ_FIELD_IQ2_BLOCK &&
      ((uintptr_t)(dst + i) % 8) == 0) {
    uint64_t w = mix64(key + (p0 / 8 + 1) * 0x9E3779B97F4A7C15ull);
    uint64_t o = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      uint32_t b = (uint32_t)(w >> (8 * j)) & 0xFFu;
      o |= (uint64_t)map_byte(key, p0 + j, b, field, dtab) << (8 * j);
    }
    *reinterpret_cast<uint64_t*>(dst + i) = o;
    return;
  }
  for (int j = 0; j < 8 && i + j < nbytes; j++) {
    uint64_t pos = p0 + j;
    dst[i + j] = (uint8_t)map_byte(key, pos, raw_byte(key, pos), field, dtab);
  }
}

}  // namespace

extern "C" int moeq_synth_fill(uint8_t* dst, size_t nbytes, uint64_t seed, uint32_t stream, uint64_t byte_offset,
                               int field, const uint16_t* d_table, void* hip_stream) {
  if (field < MOEQ_FIELD_RAW || field > MOEQ_FIELD_IQ2_BLOCK) return MOEQ_E_INVAL;
  if (nbytes == 0) return MOEQ_OK;
  if (!dst) return MOEQ_E_INVAL;
  if (field == MOEQ_FIELD_Q2K_BLOCK || field == MOEQ_FIELD_IQ2_BLOCK) {
    const uint64_t bs = field == MOEQ_FIELD_Q2K_BLOCK ? 84 : 66;
    if (!d_table || byte_offset % bs || nbytes % bs) return MOEQ_E_INVAL;
  }
  const uint64_t key = mix64(((seed & 0xFFFFFFFFull) << 32) | (uint64_t)stream);
  const size_t threads = (nbytes + 7) / 8;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, (hipStream_t)hip_stream, dst,
                     nbytes, key, byte_offset, field, d_table);
  return hipGetLastError() == hipSuccess ? MOEQ_OK : MOEQ_E_HIP;
}
