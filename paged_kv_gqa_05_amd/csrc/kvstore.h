#pragma once
// Writing one element of the paged KV cache: the tile layouts (include/pkv.h)
// and the E4M3 code of a value for quantised caches (rvLLM post on
// discuss.pytorch.kr, section "PagedAttention과 FlashAttention-3": FP8 E4M3 KV
// cache; format: OCP E4M3FN, one float32 scale per layer and tensor).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// E4M3 code of x: the nearest representable value, ties to the even code,
// magnitudes at or above the largest finite value (448) saturated to it, NaN
// to 0x7F with the sign of x.  Below 2^-6 the format steps by 2^-9
// (subnormals); above, an exponent e = floor(log2 |x|) leaves 3 mantissa
// bits, i.e. steps of 2^(e-3).  rintf rounds to nearest even.
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80;
  const float a = fabsf(x);
  if (!(a == a)) return (uint8_t)(sign | 0x7F);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
  int code;
  if (a < 0.015625f) {
    code = (int)rintf(a * 512.0f);  // 0 .. 8; 8 is the smallest normal (code 0x08)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
    const int q = (int)rintf(ldexpf(a, 3 - e));                    // 8 .. 16
    code = ((e + 7) << 3) + q - 8;  // q == 16 carries into the next exponent
  }
  return (uint8_t)(sign | code);
}

// Offset of (token slot t, dim d) inside one [BS = 16]-token tile, in elements.
__device__ __forceinline__ int k_tile_off(bool fp8, int t, int d) {
  return fp8 ? ((d >> 4) * 16 + t) * 16 + (d & 15) : ((d >> 3) * 16 + t) * 8 + (d & 7);
}
__device__ __forceinline__ int v_tile_off(bool fp8, int t, int d) {
  return fp8 ? ((((d >> 6) * 4 + (t >> 2)) * 16 + (d & 15)) * 16 + ((d >> 4) & 3) * 4 + (t & 3)) : d * 16 + t;
}

// Stores x (rounded to f16, the precision of the new token's k and v) at
// element `off` of a pool: as f16, or as the E4M3 code of f16(x) / scale with
// the quotient formed in float32.  One token fills only 1-2 bytes of every 32
// bytes of a K or V tile, so the store writes through L2 (agent scope):
// leaving such lines partly dirty in L2 until the end of the kernel cost the
// QKV projection at batch 256 about 1 us more per layer.
__device__ __forceinline__ void kv_store(void* pool, size_t off, bool fp8, float scale, float x) {
  const _Float16 h = (_Float16)x;
  if (fp8)
    __hip_atomic_store(static_cast<uint8_t*>(pool) + off, e4m3_encode(__fdiv_rn((float)h, scale)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(static_cast<unsigned short*>(pool) + off, __builtin_bit_cast(unsigned short, h),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace pkv
