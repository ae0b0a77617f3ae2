// Packed key/value tiles and direct global->LDS copy helpers.
#pragma once
#include "nsa_common.h"

namespace nsa {

// Packed block layout shared by global memory and LDS (the tiles are
// copied verbatim by direct global->LDS loads): K tile [64 keys][D] then
// V^T tile [D dims][64 keys], 16-byte chunks (8 elements) permuted per row.
// A fragment read by lanes 0..15 (16 consecutive rows, one chunk index)
// then touches 16 distinct 16-byte bank groups.
template <int D>
struct PackedTile {
  static constexpr int KE = kBlk * D, VE = D * kBlk;  // elements
  // chunk position of logical chunk c in row r of a row of `bytes` bytes
  template <int BYTES>
  __host__ __device__ static constexpr int swz(int r, int c) {
    return BYTES >= 256 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
  }
  // V^T rows hold each 32-key half with keys permuted so that lane group j
  // of the PV fragment finds its eight keys {4j..4j+3, 16+4j..16+4j+3} in
  // one chunk: stored key slot 8j+i <- key 4j+i (i < 4), 16+4j+i-4 (i >= 4)
  __host__ __device__ static constexpr int vkey(int slot) {
    const int h = slot / 32, p = slot % 32, j = p / 8, i = p % 8;
    return 32 * h + (i < 4 ? 4 * j + i : 16 + 4 * j + (i - 4));
  }
  // the stored slot of key `key` (inverse of vkey)
  __host__ __device__ static constexpr int vslot(int key) {
    const int h = key / 32, q = key % 32, r = q & 15;
    return 32 * h + 8 * (r / 4) + (r % 4) + (q >= 16 ? 4 : 0);
  }
};

// A operand of S^T = K Q^T from a staged K tile: keys 16*kt + (l%16), dims
// 32*ds + 8*(l/16) .. +7.
template <int D>
__device__ __forceinline__ u16x8 pk_k_frag(const uint16_t *ks, int kt, int ds, int lane) {
  const int r = 16 * kt + (lane & 15), c = 4 * ds + (lane >> 4);
  return *reinterpret_cast<const u16x8 *>(ks + r * D + 8 * PackedTile<D>::template swz<2 * D>(r, c));
}
// A operand of O^T = V^T P^T from a staged V^T tile: dim 16*dt + (l%16),
// the eight keys of lane group l/16 in half ks (one swizzled chunk).
template <int D>
__device__ __forceinline__ u16x8 pk_v_frag(const uint16_t *vt, int dt, int ks, int lane) {
  const int r = 16 * dt + (lane & 15), c = 4 * ks + (lane >> 4);
  return *reinterpret_cast<const u16x8 *>(vt + r * kBlk + 8 * PackedTile<D>::template swz<2 * kBlk>(r, c));
}

// Waits until at most N vector-memory operations of this wave are in flight
// (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, other counters at max).
template <int N> __device__ __forceinline__ void wait_vm_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Waits until at most n blocks of PPP copies each are still in flight.
template <int PPP>
__device__ __forceinline__ void wait_blocks(int n) {
  switch (n) {
    case 0: wait_vm_c<0>(); break;
    case 1: wait_vm_c<PPP>(); break;
    case 2: if constexpr (2 * PPP < 64) wait_vm_c<2 * PPP>(); else wait_vm_c<0>(); break;
    case 3: if constexpr (3 * PPP < 64) wait_vm_c<3 * PPP>(); else wait_vm_c<0>(); break;
    case 4: if constexpr (4 * PPP < 64) wait_vm_c<4 * PPP>(); else wait_vm_c<0>(); break;
    case 5: if constexpr (5 * PPP < 64) wait_vm_c<5 * PPP>(); else wait_vm_c<0>(); break;
    case 6: if constexpr (6 * PPP < 64) wait_vm_c<6 * PPP>(); else wait_vm_c<0>(); break;
    default: wait_vm_c<0>(); break;
  }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) int lds_int;
// Uncached LDS accesses of the protocol counters (explicitly in the LDS
// address space, so they are ds_* instructions and never wait on the copies)
__device__ __forceinline__ int lds_load(int *p) { return *(volatile lds_int *)(p); }
__device__ __forceinline__ void lds_store(int *p, int v) { *(volatile lds_int *)(p) = v; }

// Issues NP pieces of 1 KB (512 16-bit elements) from src to dst as direct
// global->LDS copies (each lane moves 16 bytes per piece), four pieces per
// address set-up (immediate offsets 0..3 KB).
template <int NP>
__device__ __forceinline__ void dma_pieces(const uint16_t *src, uint16_t *dst, int lane) {
#pragma unroll
  for (int q0 = 0; q0 < NP; q0 += 4) {
    const uint16_t *s4 = src + q0 * 512 + lane * 8;
    lds_void *d4 = (lds_void *)(dst + q0 * 512);
    __builtin_amdgcn_global_load_lds(s4, d4, 16, 0, 0);
    if (q0 + 1 < NP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 1024, 0);
    if (q0 + 2 < NP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 2048, 0);
    if (q0 + 3 < NP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 3072, 0);
  }
}

// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence would wait for every copy still in flight); callers order their own
// copies with explicit vmcnt waits.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace nsa
