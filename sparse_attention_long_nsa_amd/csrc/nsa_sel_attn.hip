// Selection branch: every vision query attends to the tokens of the blocks
// chosen for it (VideoNSA paper summary page, "Method", branch (b)); the
// query's own block is causal inside.
//
// Selected blocks differ per query, and only the G query heads of one token
// share a set, so a 16-row matrix-core tile holds TP = 16/G tokens x G heads.
// One workgroup takes one 64-token frame and one KV group: it builds the
// union of the blocks its tokens selected (tokens of a frame pick largely the
// same blocks), walks the union in ascending order staging each block's K
// and V^T into LDS once, and runs only the tiles that picked that block.
// Blocks arrive by direct global->LDS loads into a three-slot ring, issued
// two blocks ahead, so the gather latency hides behind the matrix work
// without holding any staging registers. Values are first packed once per
// call into a block-major, transposed fp16 copy so that those loads are
// plain linear copies.
#include "nsa_kernels.h"

namespace nsa {

namespace {

constexpr int kSelMaxK = 64;
constexpr int kSelMaxBlk = 8192;
constexpr int kRing = 3;  // LDS block buffers: prefetch distance 2

constexpr int kSelTok = 32;  // tokens per workgroup: half a frame

template <int D, int G>
struct SelCfg {
  static constexpr int TP = 16 / G;                       // tokens per row tile
  static constexpr int NRT = (kSelTok + TP - 1) / TP;     // row tiles per workgroup
  static constexpr int RT = 1;                            // row tiles per wave
  static constexpr int NW = (NRT + RT - 1) / RT;          // waves
  static constexpr int NT = 64 * NW;                      // threads
  // LDS tiles use the padded, conflict-free layouts of Tile<D>, rounded up
  // to whole 1-KB DMA pieces (512 elements).
  static constexpr int KP = (Tile<D>::kElems + 511) / 512;  // pieces of a K tile
  static constexpr int VP = (Tile<D>::vElems + 511) / 512;  // pieces of a V^T tile
  static constexpr int KE = KP * 512, VE = VP * 512;        // tile sizes (elements)
  static constexpr int KRW = (kBlk + NW - 1) / NW;          // K rows per wave (max)
  static constexpr int VPW = (VP + NW - 1) / NW;            // V^T pieces per wave (max)
};

// Waits until at most n (0..63) vector-memory operations of this wave are in
// flight (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, other counters
// at their maximum).
template <int N> __device__ __forceinline__ void wait_vm_c() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: wait_vm_c<0>(); break;   case 1: wait_vm_c<1>(); break;
    case 2: wait_vm_c<2>(); break;   case 3: wait_vm_c<3>(); break;
    case 4: wait_vm_c<4>(); break;   case 5: wait_vm_c<5>(); break;
    case 6: wait_vm_c<6>(); break;   case 7: wait_vm_c<7>(); break;
    case 8: wait_vm_c<8>(); break;   case 9: wait_vm_c<9>(); break;
    case 10: wait_vm_c<10>(); break; case 11: wait_vm_c<11>(); break;
    case 12: wait_vm_c<12>(); break; case 13: wait_vm_c<13>(); break;
    case 14: wait_vm_c<14>(); break; case 15: wait_vm_c<15>(); break;
    case 16: wait_vm_c<16>(); break; case 17: wait_vm_c<17>(); break;
    case 18: wait_vm_c<18>(); break; case 20: wait_vm_c<20>(); break;
    case 24: wait_vm_c<24>(); break; case 32: wait_vm_c<32>(); break;
    case 40: wait_vm_c<40>(); break; case 48: wait_vm_c<48>(); break;
    default: wait_vm_c<0>(); break;
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Issues one block as direct global->LDS loads. K: one instruction per row;
// the DMA writes 4 bytes per lane at lane*4, so the first D/2 lanes copy one
// row into the padded [64][D+8] tile at a uniform LDS address (rows past the
// data repeat row 0; those keys are masked). V^T: the packed block is copied
// linearly in 1-KB pieces. Wave wv moves rows wv, wv+NW, ... and pieces wv,
// wv+NW, ...
template <int D, int G>
__device__ __forceinline__ void dma_block(uint16_t *ks, uint16_t *vt, const uint16_t *kb, int64_t kstride,
                                          int nvalid, const uint16_t *vtb, int wv, int lane) {
  using C = SelCfg<D, G>;
  constexpr int KS = Tile<D>::kStr;
#pragma unroll
  for (int i = 0; i < C::KRW; ++i) {
    const int r = wv + i * C::NW;
    if (r < kBlk && lane < D / 2) {
      const int rr = r < nvalid ? r : 0;
      __builtin_amdgcn_global_load_lds(kb + rr * kstride + lane * 2, (lds_void *)(ks + r * KS), 4, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < C::VPW; ++i) {
    const int vp = wv + i * C::NW;
    if (vp < C::VP)
      __builtin_amdgcn_global_load_lds(vtb + vp * 512 + lane * 8, (lds_void *)(vt + vp * 512), 16, 0, 0);
  }
}

template <int D, int G>
struct SelState {
  u16x8 qf[SelCfg<D, G>::RT][D / 32];
  f32x4 o[SelCfg<D, G>::RT][D / 16];
  float m[SelCfg<D, G>::RT], l[SelCfg<D, G>::RT];
  int cur[SelCfg<D, G>::RT][SelCfg<D, G>::TP];
};

// Consumes one staged block b for the wave's tiles.
template <int D, int G, bool F16>
__device__ __forceinline__ void sel_block(SelState<D, G> &st, const uint16_t *ks, const uint16_t *vt,
                                          const int32_t *sl, int b, int k, int tok0, int ntok,
                                          float sl2, int wv, int lane) {
  using C = SelCfg<D, G>;
  constexpr int TP = C::TP, RT = C::RT, NRT = C::NRT;
  const int grp = lane >> 4, r16 = lane & 15, tau = r16 / G;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int ti = wv * RT + r;
    if (ti >= NRT) continue;
    uint32_t needmask = 0;
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      const int tk = ti * TP + i;
      if (tk < ntok && st.cur[r][i] < k) {
        const int sb = __builtin_amdgcn_readfirstlane(sl[tk * k + st.cur[r][i]]);
        if (sb == b) { needmask |= 1u << i; ++st.cur[r][i]; }
      }
    }
    if (needmask == 0) continue;
    const int tk = ti * TP + tau;
    const bool rowneed = tau < TP && tk < ntok && ((needmask >> tau) & 1u);
    const int t = tok0 + tk;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      f32x4 s[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kt = 2 * ks2 + kk;
        s[kk] = zero4();
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) s[kk] = mfma_qk<F16>(k_frag<D>(ks, kt, ds, lane), st.qf[r][ds], s[kk]);
        const int j0 = b * kBlk + 16 * kt + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kk][i] = (rowneed && j0 + i <= t) ? s[kk][i] * sl2 : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = grp_max(mx);
      const float mn = fmaxf(st.m[r], mx);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(st.m[r] - mn);
      const float base = (mn == -INFINITY) ? 0.f : mn;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kk][i] = exp2f(s[kk][i] - base);
      st.l[r] = st.l[r] * alpha + (s[0][0] + s[0][1] + s[0][2] + s[0][3]) + (s[1][0] + s[1][1] + s[1][2] + s[1][3]);
      st.m[r] = mn;
      const u16x8 pp = pack_p(s[0], s[1]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) st.o[r][dt] = mfma_f16(v_frag<D>(vt, dt, ks2, lane), pp, st.o[r][dt] * alpha);
    }
  }
}

template <int D, int G, bool F16>
__global__ __launch_bounds__((SelCfg<D, G>::NT)) void sel_attn_kernel(SelParams p) {
  using C = SelCfg<D, G>;
  constexpr int TP = C::TP, RT = C::RT, NRT = C::NRT, NT = C::NT;
  // three ring slots as separate LDS objects, so that reads of one slot need
  // not wait for loads still landing in another
  __shared__ __attribute__((aligned(16))) uint16_t k0[C::KE], k1[C::KE], k2[C::KE];
  __shared__ __attribute__((aligned(16))) uint16_t v0_[C::VE], v1_[C::VE], v2_[C::VE];
  __shared__ int32_t sl[kSelTok * kSelMaxK];
  __shared__ uint32_t ubits[kSelMaxBlk / 32 + 1];
  __shared__ int32_t ulist[kSelTok * kSelMaxK];
  __shared__ int n_union;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4;
  // Workgroup -> (KV group, frame, half): both halves of a frame go to ids 8
  // apart, i.e. to the same XCD at about the same time, so the blocks their
  // unions share are served from that XCD's L2; heaviest frames first.
  const unsigned i = blockIdx.x;
  const unsigned half = (i >> 3) & 1u;
  const unsigned rest = ((i >> 4) << 3) | (i & 7u);
  const int g = (int)(rest % p.hkv);
  const int fr = (int)(rest / p.hkv);
  if (fr >= p.n_frames) return;
  const int f = p.n_frames - 1 - fr;
  const int tok0 = f * kBlk + (int)half * kSelTok;
  const int ntok = min(kSelTok, p.n_vis - tok0);
  if (ntok <= 0) return;
  const int k = p.topk;
  const int64_t kvs = (int64_t)p.hkv * D;

  // selected blocks of the workgroup's queries, and their union as a bitmask
  const int nwords = f / 32 + 1;
  for (int i2 = tid; i2 < nwords; i2 += NT) ubits[i2] = 0u;
  for (int idx = tid; idx < kSelTok * k; idx += NT) {
    const int tk = idx / k;
    sl[idx] = tk < ntok ? p.sel[((int64_t)(tok0 + tk) * p.hkv + g) * k + (idx % k)] : -1;
  }
  __syncthreads();
  for (int idx = tid; idx < kSelTok * k; idx += NT) {
    const int b = sl[idx];
    if (b >= 0 && b <= f) atomicOr(&ubits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  if (wv == 0) {  // compact the bitmask into an ascending list
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
      while (bits) {
        const int b = __ffs(bits) - 1;
        ulist[o++] = wi * 32 + b;
        bits &= bits - 1;
      }
      running += __shfl(incl, 63);
    }
    if (lane == 0) n_union = running;
  }
  __syncthreads();
  const int nU = n_union;

  const uint16_t *kbase = p.k + (p.v0 * p.hkv + g) * (int64_t)D;
  const uint16_t *vtg = p.vt + (int64_t)g * p.n_frames * C::VE;
  auto issue = [&](uint16_t *ks, uint16_t *vt, int u) {
    const int b = ulist[u];
    dma_block<D, G>(ks, vt, kbase + (int64_t)b * kBlk * kvs, kvs, min(kBlk, p.n_vis - b * kBlk),
                    vtg + (int64_t)b * C::VE, wv, lane);
  };
  if (nU > 0) issue(k0, v0_, 0);
  if (nU > 1) issue(k1, v1_, 1);

  SelState<D, G> st;
  {
    const int r16 = lane & 15, tau = r16 / G, hh = r16 % G;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int ti = wv * RT + r;
      const int tk = ti * TP + tau;
      const bool valid = ti < NRT && tau < TP && tk < ntok;
      const int64_t qrow = (p.v0 + (valid ? tok0 + tk : 0)) * p.hq + (int64_t)g * G + hh;
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds)
        st.qf[r][ds] = valid ? q_frag_global(p.q + qrow * D, ds, lane) : zero8();
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) st.o[r][dt] = zero4();
      st.m[r] = -INFINITY;
      st.l[r] = 0.f;
#pragma unroll
      for (int i = 0; i < TP; ++i) st.cur[r][i] = 0;
    }
  }

  // DMA instructions this wave issues per block
  const int my_pieces = (kBlk - wv + C::NW - 1) / C::NW + (C::VP - wv + C::NW - 1) / C::NW;
  // one ring step: wait for block u, free slot (u+2)%3 by the barrier, refill
  // it two blocks ahead, consume block u. The barrier carries no memory
  // fence (that would drain the loads still in flight); the DMA is covered by
  // the explicit vmcnt wait, and every LDS read of the previous block has
  // completed before its matrix op issued.
#define NSA_SEL_STEP(KC, VC, KN, VN)                                              \
  {                                                                               \
    wait_vm(u + 1 < nU ? my_pieces : 0);                                          \
    asm volatile("" ::: "memory");                                                \
    __builtin_amdgcn_s_barrier();                                                 \
    asm volatile("" ::: "memory");                                                \
    if (u + 2 < nU) issue(KN, VN, u + 2);                                         \
    sel_block<D, G, F16>(st, KC, VC, sl, ulist[u], k, tok0, ntok, p.sl2, wv, lane); \
    if (++u >= nU) break;                                                         \
  }
  int u = 0;
  while (u < nU) {
    NSA_SEL_STEP(k0, v0_, k2, v2_)
    NSA_SEL_STEP(k1, v1_, k0, v0_)
    NSA_SEL_STEP(k2, v2_, k1, v1_)
  }
#undef NSA_SEL_STEP

  const int r16 = lane & 15, tau = r16 / G, hh = r16 % G;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float L = grp_sum(st.l[r]);
    const int ti = wv * RT + r;
    const int tk = ti * TP + tau;
    if (ti < NRT && tau < TP && tk < ntok) {
      const int64_t qrow = (p.v0 + tok0 + tk) * p.hq + (int64_t)g * G + hh;
      const float gate = sigmoidf_(p.gates[qrow * 3 + 1]) / L;
      float *dst = p.out + qrow * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        f32x4 *d4 = reinterpret_cast<f32x4 *>(dst + 16 * dt);
        *d4 = *d4 + st.o[r][dt] * gate;
      }
    }
  }
}

// Packs the values of one KV head into the selection kernel's block layout:
// per block the padded V^T tile of Tile<D> ([d][64 + 4] fp16, pads zero),
// rounded up to whole 1-KB pieces; keys past the sequence are zero.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pack_vt_kernel(const uint16_t *__restrict__ v, int64_t v0,
                                                      int n_vis, int hkv, int n_frames,
                                                      uint16_t *__restrict__ vt) {
  constexpr int VE = ((Tile<D>::vElems + 511) / 512) * 512;
  constexpr int VS = Tile<D>::vStr;
  __shared__ uint16_t tile[kBlk][D + 2];
  const int b = blockIdx.x / hkv, g = blockIdx.x % hkv;
  const int tid = threadIdx.x;
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
  uint16_t *dst = vt + ((int64_t)g * n_frames + b) * VE;
  for (int idx = tid; idx < VE; idx += 256) {
    const int d = idx / VS, key = idx % VS;
    dst[idx] = (d < D && key < kBlk) ? tile[key][d] : 0;
  }
}

template <int D, int G, bool F16>
hipError_t run_sel(const SelParams &p, hipStream_t st) {
  const unsigned n = (unsigned)p.n_frames * (unsigned)p.hkv;
  if (n == 0) return hipSuccess;
  // two halves per (frame, group), ids padded to whole groups of 16
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

hipError_t launch_pack_vt(const SelParams &p, int d, bool f16, hipStream_t st) {
  const unsigned n = (unsigned)p.n_frames * (unsigned)p.hkv;
  if (n == 0) return hipSuccess;
  if (d == 64) {
    if (f16) hipLaunchKernelGGL((pack_vt_kernel<64, true>), dim3(n), dim3(256), 0, st, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.vt);
    else hipLaunchKernelGGL((pack_vt_kernel<64, false>), dim3(n), dim3(256), 0, st, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.vt);
  } else {
    if (f16) hipLaunchKernelGGL((pack_vt_kernel<128, true>), dim3(n), dim3(256), 0, st, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.vt);
    else hipLaunchKernelGGL((pack_vt_kernel<128, false>), dim3(n), dim3(256), 0, st, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.vt);
  }
  return hipGetLastError();
}

}  // namespace nsa
