// Selection branch: every vision query attends to the tokens of the blocks
// chosen for it (VideoNSA paper summary page, "Method", branch (b)); the
// query's own block is causal inside.
//
// Selected blocks differ per query, and only the G query heads of one token
// share a set, so a 16-row matrix-core tile holds TP = 16/G tokens x G heads;
// a consumer wave owns RT such tiles. A workgroup takes TOK consecutive
// tokens (half a 64-token frame where the tiles allow: tokens of one frame
// pick largely the same blocks) of one KV group and the union of the blocks
// they selected, in ascending order. Two producer waves stream the union's
// blocks into a ring of LDS slots with direct global->LDS copies; each
// consumer wave walks the union positions its own tokens selected, waits
// only for those blocks, and runs at its own pace: there is no workgroup
// barrier per block, so a block that few tiles need costs only those tiles.
// A slot is refilled once every consumer has moved past its block. Keys and
// values are first packed once per call into block-major tiles, exactly as
// they sit in LDS (K row-major, V transposed to fp16, both with 16-byte
// chunks XOR-swizzled per row so that the 16-byte fragment reads are free of
// bank conflicts without padding), so each block is one contiguous 2*64*d
// element region and the copies are plain linear ones.
//
// Producer/consumer protocol (all counters in LDS, each written by one wave):
//   ready[p]  blocks 0..ready[p]-1 of producer p's pieces are in LDS
//   pass[c]   consumer c no longer reads blocks 0..pass[c]-1
// Producer p issues block j into slot j % R once min(pass) >= j - R + 1, and
// publishes a block after waiting for its own copies (in-order vmcnt).
// Every wait is a bounded spin, so a broken protocol ends the kernel with
// NaN outputs instead of a hang.
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kSelMaxK = 64;
constexpr int kSelMaxBlk = 8192;
constexpr int kSpinLimit = 1 << 22;   // s_sleep(1) rounds, about 0.1 s
constexpr float kRescaleSlack = 8.f;  // log2 units a running max may lag behind

template <int D, int G>
struct SelCfg {
  static constexpr int TP = 16 / G;                   // tokens per row tile
  static constexpr int RT = (TP <= 4) ? 2 : 1;        // row tiles per consumer wave
  static constexpr int TT = RT * TP;                  // tokens per consumer wave
  static constexpr int NC = (32 / TT > 0) ? 32 / TT : 1;  // consumer waves
  static constexpr int TOK = NC * TT;                 // tokens per workgroup
  static constexpr int NPW = 2;                       // producer waves
  static constexpr int NW = NC + NPW;
  static constexpr int NT = 64 * NW;
  static constexpr int KE = PackedTile<D>::KE, VE = PackedTile<D>::VE;
  static constexpr int SE = KE + VE;                  // one slot (elements)
  static constexpr int NP = SE / 512;                 // 1-KB copy pieces per block
  static constexpr int PPP = NP / NPW;                // pieces per producer per block
  static constexpr int R = (D == 64) ? 8 : 4;         // ring slots
  static constexpr int INFL = (63 / PPP < R) ? 63 / PPP : R;  // blocks in flight per producer
  static_assert(NP % NPW == 0 && PPP % 4 == 0, "pieces split evenly, four per address set-up");
  static_assert(TOK <= 32 && NW <= 16, "workgroup shape");
};

// Consumes one staged block for one row tile: S^T = K Q^T, causal mask in
// the own block, lazily rescaled softmax, O^T += V^T P^T.
template <int D, int G, bool F16>
__device__ __forceinline__ void sel_tile(const uint16_t *ks, const uint16_t *vt, const u16x8 (&qf)[D / 32],
                                         f32x4 (&o)[D / 16], float &m, float &l, bool rowneed,
                                         int mask_b, int t, float sl2, int lane) {
  const int grp = lane >> 4;
  // dims outer, key subtiles inner (two at a time): independent accumulators
  // keep the matrix pipe fed while the next fragments load
  f32x4 s[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) s[kt] = zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
#pragma unroll
    for (int k0 = 0; k0 < 4; k0 += 2) {
      u16x8 kf[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[kt] = pk_k_frag<D>(ks, k0 + kt, ds, lane);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[k0 + kt] = mfma_qk<F16>(kf[kt], qf[ds], s[k0 + kt]);
    }
  }
  if (mask_b >= 0) {  // causal inside the own block
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int j0 = mask_b * kBlk + 16 * kt + 4 * grp;
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
  const u16x8 pp[2] = {pack_p(s[0], s[1]), pack_p(s[2], s[3])};
  // key halves outer, dims inner: eight independent accumulators per half
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
    for (int d0 = 0; d0 < D / 16; d0 += 4) {
      u16x8 vf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vf[i] = pk_v_frag<D>(vt, d0 + i, kh, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[d0 + i] = mfma_f16(vf[i], pp[kh], o[d0 + i]);
    }
  }
}

template <int D, int G, bool F16>
__global__ __launch_bounds__((SelCfg<D, G>::NT)) void sel_attn_kernel(SelParams p) {
  using C = SelCfg<D, G>;
  constexpr int TP = C::TP, RT = C::RT, TT = C::TT, TOK = C::TOK, NC = C::NC, R = C::R;
  constexpr int kSent = 0x7fffffff;
  __shared__ __attribute__((aligned(16))) uint16_t ring[R * C::SE];
  __shared__ int16_t sl[TOK * kSelMaxK];       // selected blocks per token, -1 padded
  __shared__ int16_t ulist[TOK * kSelMaxK];    // union, ascending
  __shared__ uint32_t ubits[kSelMaxBlk / 32];  // union as a bitmask over blocks
  __shared__ int16_t wpre[kSelMaxBlk / 32];    // union entries before each bitmask word
  __shared__ int pass_[NC], ready_[C::NPW];
  __shared__ int tpos[TOK];                    // position of each token of the chunk
  __shared__ int n_union;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // Workgroup -> (KV group, chunk): chunks 2c and 2c+1 of a group (the two
  // halves of a frame) go to ids 8 apart, i.e. to the same XCD at about the
  // same time, so the blocks they both selected are served from that XCD's
  // L2; heaviest chunks first.
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

  // ---- selected blocks of the workgroup's tokens and their union
  for (int w = tid; w < nwords; w += C::NT) ubits[w] = 0u;
  if (tid < NC) pass_[tid] = 0;
  if (tid < C::NPW) ready_[tid] = 0;
  if (tid < TOK) tpos[tid] = tid < ntok ? (int)row_pos(p.vmap, p.v0, tok0 + tid) : 0;
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
  const int nU = n_union;

  if (wv >= NC) {
    // ---------------------------------------------------------- producer
    // producer pw moves the contiguous pieces [pw*PPP, (pw+1)*PPP) of each
    // block, four per address set-up (immediate offsets of 0..3 KB)
    const int pw = __builtin_amdgcn_readfirstlane(wv - NC);
    const uint16_t *kvg = p.kv + (int64_t)g * p.n_frames * C::SE + pw * C::PPP * 512;
    int issued = 0, pub = 0, spins = 0;
    int free_until = R - 1;  // highest block whose slot is known to be free
    // union entries of the current 64-block window and of the next one
    // (the next window is loaded a window ahead, off the critical path)
    int ul = lane < nU ? (int)ulist[lane] : 0;
    int ul_next = 64 + lane < nU ? (int)ulist[64 + lane] : 0;
    // The consumers' pass counters are read one check ahead: the LDS load
    // for the next check is issued as soon as the previous one is consumed,
    // so its latency overlaps the copies and the waits in between.
    int pv = lane < NC ? lds_load(&pass_[lane]) : kSent;
    while (pub < nU) {
      if (issued < nU && issued - pub < C::INFL) {
        if (issued > free_until) {
          int mn = pv;
#pragma unroll
          for (int q = 0; q < NC; ++q) mn = min(mn, __builtin_amdgcn_readlane(pv, q));
          free_until = __builtin_amdgcn_readfirstlane(mn + R - 1);
          pv = lane < NC ? lds_load(&pass_[lane]) : kSent;
        }
        if (issued <= free_until) {
          if (issued > 0 && (issued & 63) == 0) {
            ul = ul_next;
            ul_next = issued + 64 + lane < nU ? (int)ulist[issued + 64 + lane] : 0;
          }
          const int blk = __builtin_amdgcn_readlane(ul, issued & 63);
          const uint16_t *src = kvg + (int64_t)blk * C::SE;
          uint16_t *dst = ring + (issued % R) * C::SE + pw * C::PPP * 512;
          asm volatile("" ::: "memory");
          dma_pieces<C::PPP>(src, dst, lane);
          issued = __builtin_amdgcn_readfirstlane(issued + 1);
          continue;
        }
      }
      if (issued > pub) {  // publish the oldest block in flight
        wait_blocks<C::PPP>(issued - pub - 1);
        asm volatile("" ::: "memory");
        pub = __builtin_amdgcn_readfirstlane(pub + 1);
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
  const float sl2 = p.sl2;
  u16x8 qf[RT][D / 32];
  f32x4 o[RT][D / 16];
  float m[RT], l[RT];
  int trow[RT], own_b[RT][2], own_u[RT][2];
  bool rowvalid[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int tk = c * TT + r * TP + tau;
    rowvalid[r] = tau < TP && tk < ntok;
    trow[r] = tok0 + tk;
    const int64_t qrow = (int64_t)tpos[rowvalid[r] ? tk : 0] * p.hq + (int64_t)g * G + hh;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qf[r][ds] = rowvalid[r] ? q_frag_global(p.q + qrow * D, ds, lane) : zero8();
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[r][dt] = zero4();
    m[r] = -INFINITY;
    l[r] = 0.f;
    // own blocks of the tile's first and last token and their union
    // positions (-1 when absent): only these need the causal mask
    const int t0 = c * TT + r * TP;
    const int tfirst = tok0 + min(t0, ntok - 1), tlast = tok0 + min(t0 + TP, ntok) - 1;
    own_b[r][0] = tfirst / kBlk;
    own_b[r][1] = tlast / kBlk;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int b = own_b[r][e];
      const uint32_t w = ubits[b >> 5];
      const int u = ((w >> (b & 31)) & 1u) ? (int)wpre[b >> 5] + __popc(w & ((1u << (b & 31)) - 1u)) : -1;
      own_u[r][e] = __builtin_amdgcn_readfirstlane(u);
    }
  }
  // per token of the wave: lane j holds the union position of its j-th
  // selected block (ascending; sentinel past the end)
  int lst[TT], cur[TT], nxt[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int tq = c * TT + q;
    const int b = (tq < ntok && lane < k) ? sl[tq * k + lane] : -1;
    lst[q] = b < 0 ? kSent : (int)wpre[b >> 5] + __popc(ubits[b >> 5] & ((1u << (b & 31)) - 1u));
    cur[q] = 0;
    nxt[q] = __builtin_amdgcn_readlane(lst[q], 0);
  }
  bool bad = false;
  for (;;) {
    int u = kSent;
#pragma unroll
    for (int q = 0; q < TT; ++q) u = min(u, nxt[q]);
    if (u == kSent) break;
    uint32_t need[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) need[r] = 0u;
#pragma unroll
    for (int q = 0; q < TT; ++q) {
      if (nxt[q] == u) {
        need[q / TP] |= 1u << (q % TP);
        ++cur[q];
        nxt[q] = cur[q] < k ? __builtin_amdgcn_readlane(lst[q], cur[q]) : kSent;
      }
    }
    if (lane == 0) lds_store(&pass_[c], u);
    // wait for every producer's pieces of block u
    int spins = 0;
    auto min_ready = [&]() {
      int r = lds_load(&ready_[0]);
#pragma unroll
      for (int q = 1; q < C::NPW; ++q) r = min(r, lds_load(&ready_[q]));
      return r;
    };
    while (min_ready() <= u) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) { bad = true; break; }
    }
    asm volatile("" ::: "memory");
    const uint16_t *ks = ring + (u % R) * C::SE;
    const uint16_t *vt = ks + C::KE;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (need[r]) {
        const int mask_b = (u == own_u[r][0]) ? own_b[r][0] : (u == own_u[r][1]) ? own_b[r][1] : -1;
        const bool rowneed = rowvalid[r] && ((need[r] >> tau) & 1u);
        sel_tile<D, G, F16>(ks, vt, qf[r], o[r], m[r], l[r], rowneed, mask_b, trow[r], sl2, lane);
      }
    }
  }
  // all reads of ring slots have returned before the final release
  __builtin_amdgcn_s_waitcnt(0xC07F);
  if (lane == 0) lds_store(&pass_[c], nU);

  const int grp = lane >> 4;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float L = grp_sum(l[r]);
    if (rowvalid[r]) {
      const int64_t qrow = (int64_t)tpos[c * TT + r * TP + tau] * p.hq + (int64_t)g * G + hh;
      const float gate = bad ? __builtin_nanf("") : sigmoidf_(p.gates[qrow * 3 + 1]) / L;
      float *dst = p.out + qrow * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        // streaming read-modify-write of the output (non-temporal, so the
        // output does not push the key tiles out of the last-level cache)
        f32x4 *d4 = reinterpret_cast<f32x4 *>(dst + 16 * dt);
        __builtin_nontemporal_store(__builtin_nontemporal_load(d4) + o[r][dt] * gate, d4);
      }
    }
  }
}

// Packs one KV head's keys and values into the block layout (PackedTile):
// per (head, block) the swizzled K tile (as given: bf16, or fp16 for fp32
// inputs) followed by the swizzled, key-permuted V^T tile in fp16; rows past
// n_vis are zero. Packed row t reads source row rows[t] when a row map is
// given, else v0 + t, plus `jump` from row split_at on (to skip a run of
// rows, e.g. the vision run for text).
template <int D, bool F16>
__global__ __launch_bounds__(256) void pack_kv_kernel(const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v, int64_t v0,
                                                      int n_vis, int split_at, int64_t jump, int hkv,
                                                      int n_frames, uint16_t *__restrict__ kv,
                                                      const int32_t *__restrict__ rows) {
  using T = PackedTile<D>;
  __shared__ uint16_t tile[kBlk][D + 2];
  const int b = blockIdx.x / hkv, g = blockIdx.x % hkv;
  const int tid = threadIdx.x;
  uint16_t *dst = kv + ((int64_t)g * n_frames + b) * (T::KE + T::VE);
  // K: chunk c of key row r goes to chunk position swz(r, c)
  for (int idx = tid; idx < kBlk * (D / 8); idx += 256) {
    const int r = idx / (D / 8), c = idx % (D / 8);
    const int t = b * kBlk + r;
    u16x8 val = zero8();
    if (t < n_vis) {
      const int64_t src = rows ? (int64_t)rows[t] : v0 + t + (t >= split_at ? jump : 0);
      val = *reinterpret_cast<const u16x8 *>(k + (src * hkv + g) * (int64_t)D + 8 * c);
    }
    *reinterpret_cast<u16x8 *>(dst + r * D + 8 * T::template swz<2 * D>(r, c)) = val;
  }
  for (int idx = tid; idx < kBlk * D; idx += 256) {
    const int key = idx / D, d = idx % D;
    const int t = b * kBlk + key;
    uint16_t x = 0;
    if (t < n_vis) {
      const int64_t src = rows ? (int64_t)rows[t] : v0 + t + (t >= split_at ? jump : 0);
      x = v[(src * hkv + g) * (int64_t)D + d];
      if (!F16) x = bf2h_bits(x);
    }
    tile[key][d] = x;
  }
  __syncthreads();
  // V^T: row d, stored key slot s <- key vkey(s); chunk c at swz(d, c)
  for (int idx = tid; idx < D * (kBlk / 8); idx += 256) {
    const int d = idx / (kBlk / 8), c = idx % (kBlk / 8);
    u16x8 val;
#pragma unroll
    for (int i = 0; i < 8; ++i) val[i] = tile[T::vkey(8 * c + i)][d];
    *reinterpret_cast<u16x8 *>(dst + T::KE + d * kBlk + 8 * T::template swz<2 * kBlk>(d, c)) = val;
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

hipError_t launch_pack_tiles(const uint16_t *k, const uint16_t *v, int64_t row0, int n_rows, int hkv,
                             int n_chunks, uint16_t *out, int d, bool v_f16, hipStream_t st,
                             int split_at, int64_t jump, const int32_t *rows) {
  const unsigned n = (unsigned)n_chunks * (unsigned)hkv;
  if (n == 0) return hipSuccess;
  if (d == 64) {
    if (v_f16) hipLaunchKernelGGL((pack_kv_kernel<64, true>), dim3(n), dim3(256), 0, st, k, v, row0, n_rows, split_at, jump, hkv, n_chunks, out, rows);
    else hipLaunchKernelGGL((pack_kv_kernel<64, false>), dim3(n), dim3(256), 0, st, k, v, row0, n_rows, split_at, jump, hkv, n_chunks, out, rows);
  } else {
    if (v_f16) hipLaunchKernelGGL((pack_kv_kernel<128, true>), dim3(n), dim3(256), 0, st, k, v, row0, n_rows, split_at, jump, hkv, n_chunks, out, rows);
    else hipLaunchKernelGGL((pack_kv_kernel<128, false>), dim3(n), dim3(256), 0, st, k, v, row0, n_rows, split_at, jump, hkv, n_chunks, out, rows);
  }
  return hipGetLastError();
}

hipError_t launch_pack_kv(const SelParams &p, int d, bool f16, hipStream_t st) {
  return launch_pack_tiles(p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv, d, f16, st,
                           0x7fffffff, 0, p.vmap);
}

size_t packed_kv_block_elems(int d) { return (size_t)2 * kBlk * d; }

}  // namespace nsa
