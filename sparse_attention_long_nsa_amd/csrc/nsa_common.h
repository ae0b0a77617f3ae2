// Shared device helpers for the gfx950 kernels of libnsa.
//
// Matrix-core convention used by every attention kernel (CDNA3/CDNA4
// v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 x 32): lane l supplies row (l % 16), k-slots 8*(l/16) .. +7
//   B operand (32 x 16): lane l supplies column (l % 16), same k-slots
//   D (16 x 16 fp32):    lane l holds column (l % 16), rows 4*(l/16) .. +3
// Scores are computed transposed, S^T = K * Q^T (A = 16 keys x 32 dims from
// LDS, B = Q^T held in registers), so lane l owns query row (l % 16) and keys
// 4*(l/16)+i of each 16-key subtile. The probabilities of two consecutive key
// subtiles then form the B operand of O^T = V^T * P^T directly: lane group j
// uses keys {4j..4j+3} and {16+4j..16+4j+3} as its eight k-slots, and the A
// operand V^T is read with the same key order from a transposed LDS tile.
// Every per-row quantity (max, sum, output column) lives in lane l % 16.
// The k-slot order only has to agree between A and B, so it is free.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;         // compression / selection block, one key chunk
constexpr float kLog2e = 1.4426950408889634f;

// LDS tiles hold raw 16-bit elements (bf16 or fp16, as the kernel uses them).
// K tiles: [64 keys][D + 8] -> each row starts 4 banks after the previous
// one, so 8 lanes reading 16 B from 8 different keys hit 32 distinct banks.
// V^T tiles: [D][64 + 4] -> 16 lanes reading 8 B from 16 different dims hit
// 32 distinct banks.
template <int D> struct Tile {
  static constexpr int kStr = D + 8;
  static constexpr int vStr = kBlk + 4;
  static constexpr int kElems = kBlk * kStr;
  static constexpr int vElems = D * vStr;
};

// Scores: bf16 x bf16 (exact products of bf16 inputs) or fp16 x fp16.
__device__ __forceinline__ f32x4 mfma_bf16(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// Probability x value products run in fp16: probabilities lie in [0, 1] and
// fp16 keeps 11 significant bits (bf16: 8), so the PV rounding error is 8x
// smaller at the same matrix-core rate.
__device__ __forceinline__ f32x4 mfma_f16(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Scores in the operands' own type: bf16 inputs (exact products) or fp16.
template <bool F16>
__device__ __forceinline__ f32x4 mfma_qk(u16x8 a, u16x8 b, f32x4 c) {
  if constexpr (F16) return mfma_f16(a, b, c);
  else return mfma_bf16(a, b, c);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ u16x8 zero8() { return u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }

__device__ __forceinline__ float bf2f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ bf16 f2bf(float x) { return static_cast<bf16>(x); }
__device__ __forceinline__ uint16_t f2h_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<f16>(x)); }
__device__ __forceinline__ uint16_t f2bf_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<bf16>(x)); }
__device__ __forceinline__ float bfbits2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// bf16 -> fp16: exact for magnitudes in fp16's normal range.
__device__ __forceinline__ uint16_t bf2h_bits(uint16_t b) { return f2h_bits(bfbits2f(b)); }

// Reductions over the four lanes l, l^16, l^32, l^48 (one query row of a
// transposed score tile) with the row-swap permutes: the 32-lane swap of x
// with itself yields x[l mod 32] and x[(l mod 32) + 32] in the two results,
// the 16-lane swap likewise pairs rows 0/1 and 2/3.
// Maximum of two floats that are never NaN, as one v_med3_f32 against +inf:
// med3(a, b, +inf) = max(a, b). fmaxf instead costs up to three
// instructions, since LLVM quiets each operand it cannot prove canonical
// (matrix-core and permute results) with a v_max_f32 x, x, x first. The +inf
// comes from an opaque scalar move so that LLVM does not rewrite the med3
// back into fmaxf's form.
__device__ __forceinline__ float pos_inf_opaque() {
  float x;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(x));
  return x;
}
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, pos_inf_opaque()); }
__device__ __forceinline__ float grp_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmax_nn(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmax_nn(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float grp_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Packs eight probabilities (two f32x4 from consecutive key subtiles) into
// the fp16 B operand of the PV product.
__device__ __forceinline__ u16x8 pack_p(f32x4 a, f32x4 b) {
  return u16x8{f2h_bits(a[0]), f2h_bits(a[1]), f2h_bits(a[2]), f2h_bits(a[3]),
               f2h_bits(b[0]), f2h_bits(b[1]), f2h_bits(b[2]), f2h_bits(b[3])};
}

// ---------------------------------------------------------------- staging
// Copies up to 64 rows of D 16-bit elements (row r at src + r * src_stride)
// into an LDS K tile; rows >= n_valid are zero-filled.
template <int D>
__device__ __forceinline__ void stage_k(uint16_t *__restrict__ ks, const void *__restrict__ src_,
                                        int64_t src_stride, int n_valid, int tid, int nthr) {
  const uint16_t *src = static_cast<const uint16_t *>(src_);
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int idx = tid; idx < kBlk * CH; idx += nthr) {
    const int r = idx / CH, c = idx % CH;
    u16x8 val = zero8();
    if (r < n_valid) val = *reinterpret_cast<const u16x8 *>(src + r * src_stride + c * 8);
    *reinterpret_cast<u16x8 *>(ks + r * Tile<D>::kStr + c * 8) = val;
  }
}

// Same rows of values, written transposed into an LDS V^T tile
// (vt[dim][key]) as fp16. SRC_BF16 converts bf16 sources on the way; fp16
// sources are copied. Each thread handles a pair of keys so that every LDS
// store is one dword.
template <int D, bool SRC_BF16>
__device__ __forceinline__ void stage_vt(uint16_t *__restrict__ vt, const void *__restrict__ src_,
                                         int64_t src_stride, int n_valid, int tid, int nthr) {
  const uint16_t *src = static_cast<const uint16_t *>(src_);
  constexpr int CH = D / 8;
  for (int idx = tid; idx < (kBlk / 2) * CH; idx += nthr) {
    const int kp = idx % (kBlk / 2), c = idx / (kBlk / 2);
    const int r0 = 2 * kp;
    u16x8 a = zero8(), b = zero8();
    if (r0 < n_valid) a = *reinterpret_cast<const u16x8 *>(src + r0 * src_stride + c * 8);
    if (r0 + 1 < n_valid) b = *reinterpret_cast<const u16x8 *>(src + (r0 + 1) * src_stride + c * 8);
    uint16_t *base = vt + (c * 8) * Tile<D>::vStr + r0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = SRC_BF16 ? bf2h_bits(a[i]) : a[i];
      const uint32_t hi = SRC_BF16 ? bf2h_bits(b[i]) : b[i];
      *reinterpret_cast<uint32_t *>(base + i * Tile<D>::vStr) = lo | (hi << 16);
    }
  }
}

// --------------------------------------------------------- fragment loads
// A operand of S^T = K Q^T: keys 16*kt + (l%16), dims 32*ds + 8*(l/16) ..+7.
template <int D>
__device__ __forceinline__ u16x8 k_frag(const uint16_t *ks, int kt, int ds, int lane) {
  return *reinterpret_cast<const u16x8 *>(ks + (16 * kt + (lane & 15)) * Tile<D>::kStr +
                                          32 * ds + 8 * (lane >> 4));
}

// A operand of O^T = V^T P^T: dim 16*dt + (l%16), keys
// {32*ks + 4j .. +3} and {32*ks + 16 + 4j .. +3} with j = l/16.
template <int D>
__device__ __forceinline__ u16x8 v_frag(const uint16_t *vt, int dt, int ks, int lane) {
  const uint16_t *row = vt + (16 * dt + (lane & 15)) * Tile<D>::vStr + 32 * ks + 4 * (lane >> 4);
  const u16x4 lo = *reinterpret_cast<const u16x4 *>(row);
  const u16x4 hi = *reinterpret_cast<const u16x4 *>(row + 16);
  return u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// B operand Q^T for one query row: dims 32*ds + 8*(l/16) .. +7 of the row.
__device__ __forceinline__ u16x8 q_frag_global(const void *qrow, int ds, int lane) {
  return *reinterpret_cast<const u16x8 *>(static_cast<const uint16_t *>(qrow) + 32 * ds + 8 * (lane >> 4));
}

__device__ __forceinline__ u16x8 bf2h8(u16x8 x) {
  u16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = bf2h_bits(x[i]);
  return r;
}

// True when a 16-bit fp16 pattern is an infinity or NaN (exponent all ones):
// a value that overflowed fp16's range on conversion.
__device__ __forceinline__ bool h16_nonfinite(uint16_t h) { return (h & 0x7C00u) == 0x7C00u; }

// ------------------------------------------------------ branch partials
// Until the selection kernel writes a vision row's final output, the row's
// fp32 output slot of D floats for head h holds two fp16 partials: the gated
// compression-branch output in its first D halves (part 0) and the gated
// window-branch output in its second D halves (part 1). Each kernel writes
// only its part; the selection kernel's wave that owns the (row, head)
// reads both, adds its own gated branch and overwrites the slot with the
// fp32 sum, so the output is written once in fp32 and never read back.
// Four partial values (dims d .. d+3, d a multiple of 4) move as one 8-byte
// access of two 32-bit words, each holding two fp16 values (low half first).
template <int D>
__device__ __forceinline__ void store_partial4(float *slot, int part, int d, f32x4 v) {
  const uint2 w = {uint32_t(f2h_bits(v[0])) | (uint32_t(f2h_bits(v[1])) << 16),
                   uint32_t(f2h_bits(v[2])) | (uint32_t(f2h_bits(v[3])) << 16)};
  *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(slot) + part * D + d) = w;
}
__device__ __forceinline__ float h16_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(f16, static_cast<uint16_t>(bits & 0xffffu)));
}
template <int D>
__device__ __forceinline__ f32x4 load_partial4(const float *slot, int part, int d) {
  const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(slot) + part * D + d);
  return f32x4{h16_to_f32(w.x), h16_to_f32(w.x >> 16), h16_to_f32(w.y), h16_to_f32(w.y >> 16)};
}

}  // namespace nsa
