// Device helpers shared by the attention kernels (forward and backward):
// MFMA operand conventions, the LDS tile geometry and swizzles, the staging
// layout of one key tile, the bias tables, and scalar-load helpers.
#pragma once

#include "kernels.h"

namespace hstu {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Bias value of a masked pair. With y = s * (-alpha log2 e) + MASKED_Y finite
// and 2^y = +inf, the SiLU form y / (1 + 2^y) is exactly 0 (rcp(inf) = 0).
constexpr float MASKED_Y = 1.0e30f;
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KS = 16;  // reduction depth of one instruction
  static constexpr int HLK = 8;  // key offset of the upper half-wave: key_of(kb, v, 1) - key_of(kb, v, 0)
  using op = bf16x8;
  __device__ static inline f32x16 run(op a, op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // key (0..63 within the tile) held by accumulator register v of key block kb
  __device__ static constexpr int key_of(int kb, int v, int hl) { return kb * 32 + 16 * (v >> 3) + 8 * hl + (v & 7); }
  // physical key fed to MFMA row r of key block kb (see key_of)
  __device__ static inline int krow(int kb, int r) {
    int r16 = r & 15;
    int pr = (r16 < 4 || r16 >= 12) ? r16 : (r16 < 8 ? r16 + 4 : r16 - 4);
    return kb * 32 + (r & 16) + pr;
  }
};

template <> struct Mfma<float> {
  static constexpr int KS = 2;
  static constexpr int HLK = 4;
  using op = float;
  __device__ static inline f32x16 run(op a, op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static constexpr int key_of(int kb, int v, int hl) { return kb * 32 + 8 * (v >> 2) + 4 * hl + (v & 3); }
  __device__ static inline int krow(int kb, int r) { return kb * 32 + r; }
};

// LDS geometry of one key tile (KT rows of D elements) for element type T.
template <typename T, int D> struct Geo {
  static constexpr int EPC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                   // chunks per row (one key)
  static constexpr int ROWB = D * (int)sizeof(T);       // bytes per row
  static constexpr int TILE = KT * ROWB;                // bytes of one K (or V) tile
  static constexpr int NDMA = TILE / (NWAVES * 1024);   // 1 KB LDS DMA instructions per wave
  static constexpr int NDB = D / 32;                    // 32-wide d blocks of O
  static constexpr int NQOP = D / Mfma<T>::KS;          // Q (and K) operands per lane per key block
  static_assert(NDMA >= 1 && NDMA * NWAVES * 1024 == TILE, "tile staging map");
  // XOR swizzles on 16-byte chunks, chosen so that every 256-byte LDS access
  // window of an operand read touches 64 distinct banks. K: 16 lanes read 16
  // different rows at one chunk. V (bf16): 32 lanes of a transposing read
  // cover 4 consecutive rows x 64 bytes (d = 128: chunks 4db..4db+3, so the
  // row index mod 4 must move the chunk group; d = 64: two rows share a
  // window, rows r and r + 2 must differ; d = 32: one row per quarter).
  __device__ static inline int swz_k(int r) { return r % CPR; }
  __device__ static inline int swz_v(int r) {
    if constexpr (sizeof(T) == 4) return r % CPR;
    else if constexpr (D == 128) return 4 * (r & 3);
    else return (2 * r) % CPR;
  }
  __device__ static inline int k_off(int r, int c) { return r * ROWB + ((c ^ swz_k(r)) << 4); }
  __device__ static inline int v_off(int r, int c) { return r * ROWB + ((c ^ swz_v(r)) << 4); }
};

// One pipeline stage: a K tile, a V tile and the keys' timestamps.
template <typename T, int D> struct Stage {
  unsigned char k[Geo<T, D>::TILE] __attribute__((aligned(16)));
  unsigned char v[Geo<T, D>::TILE] __attribute__((aligned(16)));
  int32_t ts_lo[KT];
  int64_t ts64[KT];
};

struct Tables {
  float pos_t[MAX_NPOS];   // -log2(e) * position table
  float time_t[64];        // -log2(e) * time table, indexed by clz64(|dt| + 1)
};

__device__ inline int64_t shfl_xor64(int64_t x, int m) {
  return (int64_t)__shfl_xor((long long)x, m);
}

// Read-only data at a wave-uniform address through the constant address
// space: the compiler then emits a scalar load, whose wait does not also wait
// for the vector-memory DMA that is streaming the next key tile.
template <typename V> __device__ inline V ldc(const V* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (sizeof(V) % 4 == 0 && sizeof(V) > 8) {  // structs: copy word by word
    V out;
    const __attribute__((address_space(4))) uint32_t* q = (const __attribute__((address_space(4))) uint32_t*)(uintptr_t)p;
    uint32_t* o = (uint32_t*)&out;
    #pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / 4); ++i) o[i] = q[i];
    return out;
  } else {
    return *(const __attribute__((address_space(4))) V*)(uintptr_t)p;
  }
#else
  return *p;  // host pass of the kernel template (never executed)
#endif
}

__device__ inline int64_t uniform64(int64_t x) {
  return (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)x) |
         ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32)) << 32);
}

}  // namespace hstu
