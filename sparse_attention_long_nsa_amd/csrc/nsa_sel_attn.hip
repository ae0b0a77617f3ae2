// Selection branch: every vision query attends to the tokens of the blocks
// chosen for it (VideoNSA paper summary page, "Method", branch (b)); the
// query's own block is causal inside.
//
// Selected blocks differ per query, and only the G query heads of one token
// share a set, so a 16-row matrix-core tile holds TP = 16/G tokens x G heads,
// one tile per consumer wave. A workgroup takes TOK consecutive tokens of one
// KV group and the union of the blocks they selected, in ascending order.
// Two producer waves stream the union's blocks into a ring of LDS slots with
// direct global->LDS copies; each consumer wave jumps straight to the next
// block its own tile needs, waits only for that block, and runs at its own
// pace: there is no workgroup barrier per block, so a block that few tiles
// need costs only those tiles. A slot is refilled once every consumer has
// moved past its block. Keys and values are first packed once per call into
// block-major tiles (K as laid out in LDS, V transposed to fp16), so each
// block is one contiguous region and the copies are plain linear ones.
//
// Producer/consumer protocol (all counters in LDS, each written by one wave):
//   ready[p]  blocks 0..ready[p]-1 of producer p's pieces are in LDS
//   pass[c]   consumer c no longer reads blocks 0..pass[c]-1
// Producer p issues block j into slot j % R once min(pass) >= j - R + 1, and
// publishes a block after waiting for its own copies (in-order vmcnt).
// Every wait is a bounded spin, so a broken protocol ends the kernel with
// NaN outputs instead of a hang.
#include "nsa_kernels.h"

namespace nsa {

namespace {

constexpr int kSelMaxK = 64;
constexpr int kSelMaxBlk = 8192;
constexpr int kSpinLimit = 1 << 22;   // s_sleep(1) rounds, about 0.1 s
constexpr float kRescaleSlack = 8.f;  // log2 units a running max may lag behind

template <int D, int G>
struct SelCfg {
  static constexpr int TP = 16 / G;                          // tokens per row tile
  static constexpr int TOK = (14 * TP < 32) ? 14 * TP : 32;  // tokens per workgroup
  static constexpr int NC = (TOK + TP - 1) / TP;             // consumer waves, one tile each
  static constexpr int NPW = 2;                              // producer waves
  static constexpr int NW = NC + NPW;
  static constexpr int NT = 64 * NW;
  // LDS tiles use the padded, conflict-free layouts of Tile<D>, rounded up
  // to whole 1-KB copy pieces (512 elements).
  static constexpr int KP = (Tile<D>::kElems + 511) / 512;  // pieces of a K tile
  static constexpr int VP = (Tile<D>::vElems + 511) / 512;  // pieces of a V^T tile
  static constexpr int KE = KP * 512, VE = VP * 512;        // tile sizes (elements)
  static constexpr int SE = KE + VE;                        // one slot
  static constexpr int NP = KP + VP;                        // pieces per block
  static constexpr int PPP = NP / NPW;                      // pieces per producer per block
  static constexpr int R = (D == 64) ? 6 : 4;               // ring slots
  static constexpr int INFL = (63 / PPP < R) ? 63 / PPP : R;  // blocks in flight per producer
  static_assert(NP % NPW == 0, "pieces split evenly between the producers");
  static_assert(NW <= 16, "at most 16 waves");
};

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
    default: wait_vm_c<0>(); break;
  }
}

typedef __attribute__((address_space(3))) void lds_void;

typedef __attribute__((address_space(3))) int lds_int;
// Uncached LDS accesses of the protocol counters (explicitly in the LDS
// address space, so they are ds_* instructions and never wait on the copies)
__device__ __forceinline__ int lds_load(int *p) { return *(volatile lds_int *)(p); }
__device__ __forceinline__ void lds_store(int *p, int v) { *(volatile lds_int *)(p) = v; }

template <int D, int G, bool F16>
__global__ __launch_bounds__((SelCfg<D, G>::NT)) void sel_attn_kernel(SelParams p) {
  using C = SelCfg<D, G>;
  constexpr int TP = C::TP, TOK = C::TOK, NC = C::NC, R = C::R;
  constexpr int UW = TOK * kSelMaxK / 32;      // words of a union-position bitmap
  __shared__ __attribute__((aligned(16))) uint16_t ring[R * C::SE];
  __shared__ int16_t sl[TOK * kSelMaxK];       // selected blocks per token, -1 padded
  __shared__ int16_t ulist[TOK * kSelMaxK];    // union, ascending
  __shared__ uint32_t ubits[kSelMaxBlk / 32];  // union as a bitmask over blocks
  __shared__ int16_t wpre[kSelMaxBlk / 32];    // union entries before each bitmask word
  __shared__ uint32_t need_bm[TOK][UW];        // per token: union positions it selected
  __shared__ int pass_[NC], ready_[C::NPW];
  __shared__ int n_union;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  // Workgroup -> (KV group, chunk): chunks 2c and 2c+1 of a group go to ids
  // 8 apart, i.e. to the same XCD at about the same time, so the blocks they
  // both selected are served from that XCD's L2; heaviest chunks first.
  const int n_chunk = (p.n_vis + TOK - 1) / TOK;
  const int n_pair = (n_chunk + 1) / 2;
  const unsigned i = blockIdx.x;
  const unsigned odd = (i >> 3) & 1u;
  const unsigned rest = ((i >> 4) << 3) | (i & 7u);
  const int g = (int)(rest % p.hkv);
  const int pr = (int)(rest / p.hkv);
  if (pr >= n_pair) return;
  const int chunk = 2 * (n_pair - 1 - pr) + (int)odd;
  if (chunk >= n_chunk) return;
  const int tok0 = chunk * TOK;
  const int ntok = min(TOK, p.n_vis - tok0);
  const int k = p.topk;
  const int n_blk_all = (p.n_vis + kBlk - 1) / kBlk;
  const int nwords = (n_blk_all + 31) / 32;

  // ---- selected blocks of the workgroup's tokens, their union, and per
  //      token the set of union positions it needs
  for (int w = tid; w < nwords; w += C::NT) ubits[w] = 0u;
  for (int w = tid; w < TOK * UW; w += C::NT) (&need_bm[0][0])[w] = 0u;
  if (tid < NC) pass_[tid] = 0;
  if (tid < C::NPW) ready_[tid] = 0;
  for (int idx = tid; idx < TOK * k; idx += C::NT) {
    const int tk = idx / k;
    int b = tk < ntok ? p.sel[((int64_t)(tok0 + tk) * p.hkv + g) * k + (idx % k)] : -1;
    if (b >= n_blk_all) b = -1;
    sl[idx] = (int16_t)b;
  }
  __syncthreads();
  for (int idx = tid; idx < TOK * k; idx += C::NT) {
    const int b = sl[idx];
    if (b >= 0) atomicOr(&ubits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  if (wv == 0) {  // prefix counts per word and the ascending list
    int running = 0;
    for (int base = 0; base < nwords; base += 64) {
      const int wi = base + lane;
      uint32_t bits = wi < nwords ? ubits[wi] : 0u;
      const int cnt = __popc(bits);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      int o = running + incl - cnt;
      if (wi < nwords) wpre[wi] = (int16_t)o;
      while (bits) {
        const int b = __ffs(bits) - 1;
        ulist[o++] = (int16_t)(wi * 32 + b);
        bits &= bits - 1;
      }
      running += __shfl(incl, 63);
    }
    if (lane == 0) n_union = running;
  }
  __syncthreads();
  for (int idx = tid; idx < TOK * k; idx += C::NT) {
    const int b = sl[idx];
    if (b >= 0) {
      const int u = wpre[b >> 5] + __popc(ubits[b >> 5] & ((1u << (b & 31)) - 1u));
      atomicOr(&need_bm[idx / k][u >> 5], 1u << (u & 31));
    }
  }
  __syncthreads();
  const int nU = n_union;

  if (wv >= NC) {
    // ---------------------------------------------------------- producer
    // producer pw moves the contiguous pieces [pw*PPP, (pw+1)*PPP) of each
    // block, four per address set-up (immediate offsets of 0..3 KB)
    const int pw = wv - NC;
    const uint16_t *kvg = p.kv + (int64_t)g * p.n_frames * C::SE + pw * C::PPP * 512 + lane * 8;
    int issued = 0, pub = 0, spins = 0;
    while (pub < nU) {
      if (issued < nU && issued - pub < C::INFL) {
        bool free_slot = issued < R;
        if (!free_slot) {
          const int v = lane < NC ? lds_load(&pass_[lane]) : 0x7fffffff;
          free_slot = __builtin_amdgcn_ballot_w64(v < issued - R + 1) == 0;
        }
        if (free_slot) {
          const uint16_t *src = kvg + (int64_t)ulist[issued] * C::SE;
          uint16_t *dst = ring + (issued % R) * C::SE + pw * C::PPP * 512;
          asm volatile("" ::: "memory");
#pragma unroll
          for (int q0 = 0; q0 < C::PPP; q0 += 4) {
            const uint16_t *s4 = src + q0 * 512;
            lds_void *d4 = (lds_void *)(dst + q0 * 512);
            __builtin_amdgcn_global_load_lds(s4, d4, 16, 0, 0);
            if (q0 + 1 < C::PPP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 1024, 0);
            if (q0 + 2 < C::PPP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 2048, 0);
            if (q0 + 3 < C::PPP) __builtin_amdgcn_global_load_lds(s4, d4, 16, 3072, 0);
          }
          ++issued;
          continue;
        }
      }
      if (issued > pub) {  // publish the oldest block in flight
        wait_blocks<C::PPP>(issued - pub - 1);
        asm volatile("" ::: "memory");
        ++pub;
        if (lane == 0) lds_store(&ready_[pw], pub);
        asm volatile("" ::: "memory");
      } else {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {  // consumers stalled: give up, release them
          if (lane == 0) lds_store(&ready_[pw], nU);
          break;
        }
      }
    }
    return;
  }

  // ------------------------------------------------------------ consumer
  const int c = wv;
  const int r16 = lane & 15, tau = r16 / G, hh = r16 % G;
  const int tk = c * TP + tau;
  const bool rowvalid = tau < TP && tk < ntok;
  const int t = tok0 + tk;
  const int64_t qrow = (p.v0 + (rowvalid ? t : 0)) * p.hq + (int64_t)g * G + hh;
  u16x8 qf[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) qf[ds] = rowvalid ? q_frag_global(p.q + qrow * D, ds, lane) : zero8();
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = zero4();
  float m = -INFINITY, l = 0.f;
  bool bad = false;
  const float sl2 = p.sl2;

  // Own blocks of the tile's first and last token, and their union
  // positions (-1 when not in the union): only these need the causal mask.
  const int tfirst = tok0 + c * TP, tlast = tok0 + min(c * TP + TP, ntok) - 1;
  int own_b[2] = {tfirst / kBlk, tlast / kBlk}, own_u[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int b = own_b[e];
    const uint32_t w = ubits[b >> 5];
    own_u[e] = ((w >> (b & 31)) & 1u) ? (int)wpre[b >> 5] + __popc(w & ((1u << (b & 31)) - 1u)) : -1;
    own_u[e] = __builtin_amdgcn_readfirstlane(own_u[e]);
  }

  // walk the union positions the tile's tokens need, one bitmap word at a time
  const int nUW = (nU + 31) / 32;
  int wi = 0;
  uint32_t cw[TP];
#pragma unroll
  for (int q = 0; q < TP; ++q) cw[q] = (c * TP + q < ntok) ? __builtin_amdgcn_readfirstlane(need_bm[c * TP + q][0]) : 0u;
  for (;;) {
    uint32_t any = 0;
#pragma unroll
    for (int q = 0; q < TP; ++q) any |= cw[q];
    if (any == 0) {
      if (++wi >= nUW) break;
#pragma unroll
      for (int q = 0; q < TP; ++q)
        cw[q] = (c * TP + q < ntok) ? __builtin_amdgcn_readfirstlane(need_bm[c * TP + q][wi]) : 0u;
      continue;
    }
    const int bit = __ffs(any) - 1;
    const int u = wi * 32 + bit;
    uint32_t need = 0;
#pragma unroll
    for (int q = 0; q < TP; ++q) {
      need |= ((cw[q] >> bit) & 1u) << q;
      cw[q] &= ~(1u << bit);
    }
    if (lane == 0) lds_store(&pass_[c], u);
    // wait for both producers' pieces of block u
    int spins = 0;
    while (min(lds_load(&ready_[0]), lds_load(&ready_[1])) <= u) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) { bad = true; break; }
    }
    asm volatile("" ::: "memory");
    const uint16_t *ks = ring + (u % R) * C::SE;
    const uint16_t *vt = ks + C::KE;

    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = zero4();
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) s[kt] = mfma_qk<F16>(k_frag<D>(ks, kt, ds, lane), qf[ds], s[kt]);
    }
    const bool rowneed = rowvalid && ((need >> tau) & 1u);
    if (u == own_u[0] || u == own_u[1]) {  // causal inside the own block
      const int b = (u == own_u[0]) ? own_b[0] : own_b[1];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int j0 = b * kBlk + 16 * kt + 4 * grp;
#pragma unroll
        for (int e = 0; e < 4; ++e) s[kt][e] = (j0 + e <= t) ? s[kt][e] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                         fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
    const float gmx = grp_max(mx);  // all lanes take part in the exchange
    mx = rowneed ? gmx * sl2 : -INFINITY;
    // the running max only moves when a row's new max exceeds it by the
    // slack; probabilities then stay below 2^slack, exact in fp16's range
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
      m = mn;
    }
    // rows that do not take this block get probability exp2(-inf) = 0
    const float nbase = (rowneed && m != -INFINITY) ? -m : -INFINITY;
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[kt][e] = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, nbase));
        ls += s[kt][e];
      }
    l += ls;
    const u16x8 pp0 = pack_p(s[0], s[1]), pp1 = pack_p(s[2], s[3]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      o[dt] = mfma_f16(v_frag<D>(vt, dt, 0, lane), pp0, o[dt]);
      o[dt] = mfma_f16(v_frag<D>(vt, dt, 1, lane), pp1, o[dt]);
    }
  }
  // all reads of ring slots have returned before the final release
  __builtin_amdgcn_s_waitcnt(0xC07F);
  if (lane == 0) lds_store(&pass_[c], nU);

  const float L = grp_sum(l);
  if (rowvalid) {
    const float gate = bad ? __builtin_nanf("") : sigmoidf_(p.gates[qrow * 3 + 1]) / L;
    float *dst = p.out + qrow * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 *d4 = reinterpret_cast<f32x4 *>(dst + 16 * dt);
      *d4 = *d4 + o[dt] * gate;
    }
  }
}

// Packs one KV head's keys and values into the selection kernel's block
// layout: per (head, block) the padded K tile [64][d+8] (as given: bf16, or
// fp16 for fp32 inputs) followed by the padded V^T tile [d][64+4] in fp16,
// each rounded up to whole 1-KB pieces; keys past the sequence are zero.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pack_kv_kernel(const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v, int64_t v0,
                                                      int n_vis, int hkv, int n_frames,
                                                      uint16_t *__restrict__ kv) {
  constexpr int KE = ((Tile<D>::kElems + 511) / 512) * 512;
  constexpr int VE = ((Tile<D>::vElems + 511) / 512) * 512;
  constexpr int KS = Tile<D>::kStr, VS = Tile<D>::vStr;
  __shared__ uint16_t tile[kBlk][D + 2];
  const int b = blockIdx.x / hkv, g = blockIdx.x % hkv;
  const int tid = threadIdx.x;
  uint16_t *dst = kv + ((int64_t)g * n_frames + b) * (KE + VE);
  for (int idx = tid; idx < KE; idx += 256) {
    const int r = idx / KS, c = idx % KS;
    const int t = b * kBlk + r;
    dst[idx] = (r < kBlk && c < D && t < n_vis) ? k[((v0 + t) * hkv + g) * (int64_t)D + c] : 0;
  }
  for (int idx = tid; idx < kBlk * D; idx += 256) {
    const int key = idx / D, d = idx % D;
    const int t = b * kBlk + key;
    uint16_t x = 0;
    if (t < n_vis) {
      x = v[((v0 + t) * hkv + g) * (int64_t)D + d];
      if (!F16) x = bf2h_bits(x);
    }
    tile[key][d] = x;
  }
  __syncthreads();
  for (int idx = tid; idx < VE; idx += 256) {
    const int d = idx / VS, key = idx % VS;
    dst[KE + idx] = (d < D && key < kBlk) ? tile[key][d] : 0;
  }
}

template <int D, int G, bool F16>
hipError_t run_sel(const SelParams &p, hipStream_t st) {
  constexpr int TOK = SelCfg<D, G>::TOK;
  const unsigned n_chunk = (unsigned)((p.n_vis + TOK - 1) / TOK);
  if (n_chunk == 0) return hipSuccess;
  // pairs of chunks per group, ids padded to whole groups of 16
  const unsigned n = (n_chunk + 1) / 2 * (unsigned)p.hkv;
  const unsigned nwg = (2 * n + 15) / 16 * 16;
  hipLaunchKernelGGL((sel_attn_kernel<D, G, F16>), dim3(nwg), dim3(SelCfg<D, G>::NT), 0, st, p);
  return hipGetLastError();
}

template <bool F16>
hipError_t dispatch(const SelParams &p, int d, int G, hipStream_t st) {
  if (d == 64) {
    switch (G) {
      case 1: return run_sel<64, 1, F16>(p, st);
      case 2: return run_sel<64, 2, F16>(p, st);
      case 3: return run_sel<64, 3, F16>(p, st);
      case 4: return run_sel<64, 4, F16>(p, st);
      case 5: return run_sel<64, 5, F16>(p, st);
      case 6: return run_sel<64, 6, F16>(p, st);
      case 7: return run_sel<64, 7, F16>(p, st);
      case 8: return run_sel<64, 8, F16>(p, st);
    }
  } else if (d == 128) {
    switch (G) {
      case 1: return run_sel<128, 1, F16>(p, st);
      case 2: return run_sel<128, 2, F16>(p, st);
      case 3: return run_sel<128, 3, F16>(p, st);
      case 4: return run_sel<128, 4, F16>(p, st);
      case 5: return run_sel<128, 5, F16>(p, st);
      case 6: return run_sel<128, 6, F16>(p, st);
      case 7: return run_sel<128, 7, F16>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sel_attn(const SelParams &p, int d, int G, bool f16, hipStream_t st) {
  return f16 ? dispatch<true>(p, d, G, st) : dispatch<false>(p, d, G, st);
}

hipError_t launch_pack_kv(const SelParams &p, int d, bool f16, hipStream_t st) {
  const unsigned n = (unsigned)p.n_frames * (unsigned)p.hkv;
  if (n == 0) return hipSuccess;
  if (d == 64) {
    if (f16) hipLaunchKernelGGL((pack_kv_kernel<64, true>), dim3(n), dim3(256), 0, st, p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv);
    else hipLaunchKernelGGL((pack_kv_kernel<64, false>), dim3(n), dim3(256), 0, st, p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv);
  } else {
    if (f16) hipLaunchKernelGGL((pack_kv_kernel<128, true>), dim3(n), dim3(256), 0, st, p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv);
    else hipLaunchKernelGGL((pack_kv_kernel<128, false>), dim3(n), dim3(256), 0, st, p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv);
  }
  return hipGetLastError();
}

size_t packed_kv_block_elems(int d) {
  return (size_t)(((d + 8) * kBlk + 511) / 512 + (d * (kBlk + 4) + 511) / 512) * 512;
}

}  // namespace nsa
