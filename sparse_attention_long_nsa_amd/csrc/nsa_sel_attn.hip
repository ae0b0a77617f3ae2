// Selection branch: every vision query attends to the tokens of the blocks
// chosen for it (VideoNSA paper summary page, "Method", branch (b)); the
// query's own block is causal inside.
//
// Selected blocks differ per query, and only the G query heads of one token
// share a set, so a 16-row matrix-core tile holds TP = 16/G tokens x G heads;
// a consumer wave owns RT such tiles. A workgroup takes TOK consecutive
// tokens (half a 64-token frame where the tiles allow: tokens of one frame
// pick largely the same blocks) of one KV group and the union of the blocks
// they selected, in ascending order. The union's blocks pass through a ring
// of LDS slots filled by direct global->LDS copies; each wave walks the union
// positions its own tokens selected, waits only for those blocks, and runs
// at its own pace: there is no workgroup barrier per block, so a block that
// few tiles need costs only those tiles. A slot is refilled once every wave
// has moved past its block. Keys and values are first packed once per call
// into block-major tiles, exactly as they sit in LDS (K row-major, V
// transposed to fp16, both with 16-byte chunks XOR-swizzled per row so that
// the 16-byte fragment reads are free of bank conflicts without padding), so
// each block is one contiguous 2*64*d element region and the copies are
// plain linear ones.
//
// There are no copy-only waves: a wave that would wait copies instead. It
// claims the next union block whose slot every wave has left (compare-and-
// swap on a shared counter), issues the whole block's copies, waits for them
// (its own vmcnt) and publishes the block in that slot's ready word. Waves
// that are still computing leave the copying to those that are idle, and the
// workgroup is all consumers (eight waves for 7-head groups, two per SIMD,
// each with up to 256 registers). Counters, all in LDS:
//   pass[c]        wave c no longer reads union blocks 0..pass[c]-1
//   next_issue     union blocks 0..next_issue-1 have been claimed
//   ready_slot[s]  j + 1 once union block j has landed in slot s = j % R
// Block j may be claimed once min(pass) >= j - R + 1. Every wait is a
// bounded spin, so a broken protocol ends the kernel with NaN outputs and a
// flag in the workspace status word instead of a hang.
//
// Output: the (row, head) slots of the output hold the fp16 partials of the
// compression and window branches (written by their kernels); the consumer
// wave that owns a slot reads both, adds its gated selection output and
// writes the slot's final fp32 value, the only fp32 write of vision rows.
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kSelMaxK = 64;
constexpr int kSelMaxBlk = 8192;
constexpr float kRescaleSlack = 8.f;  // log2 units a running max may lag behind
constexpr uint32_t kFastMaxBits = 0x43000000u;  // bit pattern of 2^(kRescaleSlack - 1) = 128.0f

template <int D, int G>
struct SelCfg {
  static constexpr int TP = 16 / G;                   // tokens per row tile
  static constexpr int RT = (TP <= 4) ? 2 : 1;        // row tiles per consumer wave
  static constexpr int TT = RT * TP;                  // tokens per consumer wave
  static constexpr int NC = (32 / TT > 0) ? 32 / TT : 1;  // consumer waves
  static constexpr int TOK = NC * TT;                 // tokens per workgroup
  static constexpr int NW = NC;                       // waves: consumers only
  static constexpr int NT = 64 * NW;
  static constexpr int KE = PackedTile<D>::KE, VE = PackedTile<D>::VE;
  static constexpr int SE = KE + VE;                  // one slot (elements)
  static constexpr int NP = SE / 512;                 // 1-KB copy pieces per block
  static constexpr int R = (D == 64) ? 8 : 4;         // ring slots
  static_assert(NP % 4 == 0 && NP < 64, "pieces: four per address set-up, one vmcnt wait");
  static_assert(TOK <= 32 && NW <= 16, "workgroup shape");
};

// S^T = K Q^T of one staged block for one row tile, with the causal mask
// inside the own block (mask_b >= 0).
template <int D, bool F16>
__device__ __forceinline__ void sel_scores(const uint16_t *ks, const u16x8 (&qf)[D / 32], f32x4 (&s)[4],
                                           int mask_b, int t, int lane) {
  const int grp = lane >> 4;
  // dims outer, key subtiles inner (two at a time): independent accumulators
  // keep the matrix pipe fed while the next fragments load
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
}

// Probabilities 2^(s sl2 + nbase) of a tile's scores, in place, and the
// lane's share of their row sum (summed in key order).
__device__ __forceinline__ float sel_exp(f32x4 (&s)[4], float sl2, float nbase) {
  float ls = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[kt][e] = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, nbase));
      ls = (kt == 0 && e == 0) ? s[kt][e] : ls + s[kt][e];
    }
  return ls;
}

// Largest bit pattern among a lane's probabilities: they are never negative,
// so unsigned order is float order, with +inf and NaN above every finite
// value (integer maxima also need no NaN quieting and chain into v_max3_u32).
__device__ __forceinline__ uint32_t sel_max_bits(const f32x4 (&s)[4]) {
  uint32_t mb = __float_as_uint(s[0][0]);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mb = max(mb, __float_as_uint(s[kt][e]));
  return mb;
}

// Consumes one staged block for one row tile: S^T = K Q^T, causal mask in
// the own block, lazily rescaled softmax, O^T += V^T P^T.
//
// The running max m only moves when a block's scores exceed it by the slack
// (kRescaleSlack log2 units). So the probabilities are first formed against m
// as it stands, without the block max. If none exceeds 2^(slack - 1), every
// score is at least one log2 unit below m + slack (far beyond rounding): the
// full step would not move m and forms exactly these probabilities.
// Otherwise (a larger score; a row's first block, where m = -inf gives +inf;
// a masked key against an unset max, NaN) the block's scores are recomputed
// and the full step runs: block max, rescale when it exceeds m by the slack,
// probabilities. Results are bitwise those of always running the full step.
template <int D, int G, bool F16>
__device__ __forceinline__ void sel_tile(const uint16_t *ks, const uint16_t *vt, const u16x8 (&qf)[D / 32],
                                         f32x4 (&o)[D / 16], float &m, float &l, bool rowneed,
                                         int mask_b, int t, float sl2, int lane) {
  f32x4 s[4];
  sel_scores<D, F16>(ks, qf, s, mask_b, t, lane);
  float ls = sel_exp(s, sl2, rowneed ? -m : -INFINITY);
  if (__builtin_amdgcn_ballot_w64(sel_max_bits(s) > kFastMaxBits)) {
    // reload the key fragments rather than keep the first reads live
    asm volatile("" ::: "memory");
    sel_scores<D, F16>(ks, qf, s, mask_b, t, lane);
    float mx = fmax_nn(fmax_nn(fmax_nn(s[0][0], s[0][1]), fmax_nn(s[0][2], s[0][3])),
                       fmax_nn(fmax_nn(s[1][0], s[1][1]), fmax_nn(s[1][2], s[1][3])));
    mx = fmax_nn(mx, fmax_nn(fmax_nn(fmax_nn(s[2][0], s[2][1]), fmax_nn(s[2][2], s[2][3])),
                             fmax_nn(fmax_nn(s[3][0], s[3][1]), fmax_nn(s[3][2], s[3][3]))));
    const float gmx = grp_max(mx);  // all lanes take part in the exchange
    mx = rowneed ? gmx * sl2 : -INFINITY;
    // the running max only moves when a row's new max exceeds it by the
    // slack; probabilities then stay below 2^slack, exact in fp16's range
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack)) {
      const float mn = fmax_nn(m, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
      m = mn;
    }
    // rows that do not take this block get probability exp2(-inf) = 0
    ls = sel_exp(s, sl2, (rowneed && m != -INFINITY) ? -m : -INFINITY);
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
  __shared__ int pass_[NC], ready_slot[R];   // ready_slot[s]: block + 1 landed in slot s
  __shared__ int next_issue;                  // next union position to copy
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
  if (tid < R) ready_slot[tid] = 0;
  if (tid == 0) next_issue = 0;
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

  // ------------------------------------------------------------ consumer
  const int c = wv;
  const int r16 = lane & 15, tau = r16 / G, hh = r16 % G;
  const float sl2 = p.sl2;
  const uint16_t *kvg = p.kv + (int64_t)g * p.n_frames * C::SE;
  // Copies are made by consumers that would otherwise wait: claim the next
  // union block whose ring slot every consumer has left, copy it, wait for
  // this wave's own copies, publish it. False when nothing was claimable.
  auto try_copy = [&]() -> bool {
    const int j = __builtin_amdgcn_readfirstlane(lds_load(&next_issue));
    if (j >= nU) return false;
    const int pv = lane < NC ? lds_load(&pass_[lane]) : kSent;
    int mn = pv;
#pragma unroll
    for (int q = 0; q < NC; ++q) mn = min(mn, __builtin_amdgcn_readlane(pv, q));
    if (j > mn + R - 1) return false;  // its slot is still being read
    int won = 0;
    if (lane == 0) won = atomicCAS(&next_issue, j, j + 1) == j;
    if (!__builtin_amdgcn_readfirstlane(won)) return false;
    const int blk = __builtin_amdgcn_readfirstlane((int)ulist[j]);
    asm volatile("" ::: "memory");
    dma_pieces<C::NP>(kvg + (int64_t)blk * C::SE, ring + (j % R) * C::SE, lane);
    wait_vm_c<0>();
    asm volatile("" ::: "memory");
    if (lane == 0) lds_store(&ready_slot[j % R], j + 1);
    return true;
  };
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
    // wait until block u has landed in its slot, copying meanwhile
    int spins = 0;
    while (lds_load(&ready_slot[u % R]) != u + 1) {
      if (!try_copy()) __builtin_amdgcn_s_sleep(1);
      if (++spins > p.spin_limit) { bad = true; break; }
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
  if (lane == 0) {
    lds_store(&pass_[c], nU);
    if (bad && p.status) atomicOr(p.status, kStatusWaitGaveUp);  // the caller can ask
  }
  // keep copying for the consumers still walking
  for (int spins = 0; __builtin_amdgcn_readfirstlane(lds_load(&next_issue)) < nU;) {
    if (!try_copy()) __builtin_amdgcn_s_sleep(1);
    if (++spins > p.spin_limit) {
      if (lane == 0 && p.status) atomicOr(p.status, kStatusWaitGaveUp);
      break;
    }
  }

  const int grp = lane >> 4;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float L = grp_sum(l[r]);
    if (rowvalid[r]) {
      const int64_t qrow = (int64_t)tpos[c * TT + r * TP + tau] * p.hq + (int64_t)g * G + hh;
      const float gate = bad ? __builtin_nanf("") : sigmoidf_(p.gates[qrow * 3 + 1]) / L;
      float *slot = p.out + qrow * D;
      // the slot's fp16 partials of the compression and window branches,
      // read in full before the fp32 sum overwrites the slot (other lanes of
      // this wave read bytes this lane writes): all loads return first
      f32x4 part[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        part[dt] = load_partial4<D>(slot, 0, 16 * dt + 4 * grp) + load_partial4<D>(slot, 1, 16 * dt + 4 * grp);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)  // streaming (non-temporal) final write
        __builtin_nontemporal_store(part[dt] + o[r][dt] * gate,
                                    reinterpret_cast<f32x4 *>(slot + 16 * dt + 4 * grp));
    }
  }
}

// Packs one KV head's keys and values into the block layout (PackedTile):
// per (head, block) the swizzled K tile (as given: bf16, or fp16 for fp32
// inputs) followed by the swizzled, key-permuted V^T tile in fp16; rows past
// n_vis are zero. Packed row t reads source row rows[t] when a row map is
// given, else v0 + t, plus `jump` from row split_at on (to skip a run of
// rows, e.g. the vision run for text). Rows arrive as 16-byte loads, all
// issued before the first store; the values are transposed through LDS.
//
// With mk (bf16 inputs), blocks b < n_mean also yield the pooling's block
// means of their key and value columns (VideoNSA model card, "Model
// Architecture": frame blocks averaged), from the rows already in LDS, in
// the exact order of the pooling kernel's block_mean (row phases of
// 256 / (Hkv d / 8) rows, each summed in row order, then the phases in
// order, times 1/64), so the results are bitwise the pooling's own.
template <int D, bool F16>
__global__ __launch_bounds__(256) void pack_kv_kernel(const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v, int64_t v0,
                                                      int n_vis, int split_at, int64_t jump, int hkv,
                                                      int n_frames, uint16_t *__restrict__ kv,
                                                      const int32_t *__restrict__ rows, int32_t *status,
                                                      float *__restrict__ mk, float *__restrict__ mv,
                                                      int64_t n_mean) {
  using T = PackedTile<D>;
  constexpr int RS = D + 8;          // LDS row stride (16-byte rows)
  constexpr int IT = kBlk * (D / 8) / 256;  // 16-byte chunks per thread, per tensor
  __shared__ __attribute__((aligned(16))) uint16_t kt[kBlk][RS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kBlk][RS];
  __shared__ float part[2048];
  const int b = blockIdx.x / hkv, g = blockIdx.x % hkv;
  const int tid = threadIdx.x;
  const bool means = mk && b < n_mean;  // uniform over the workgroup
  uint16_t *dst = kv + ((int64_t)g * n_frames + b) * (T::KE + T::VE);
  u16x8 kx[IT], vx[IT];
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int idx = tid + 256 * j, r = idx / (D / 8), c = idx % (D / 8);
    const int t = b * kBlk + r;
    kx[j] = vx[j] = zero8();
    if (t < n_vis) {
      const int64_t src = rows ? (int64_t)rows[t] : v0 + t + (t >= split_at ? jump : 0);
      kx[j] = *reinterpret_cast<const u16x8 *>(k + (src * hkv + g) * (int64_t)D + 8 * c);
      vx[j] = *reinterpret_cast<const u16x8 *>(v + (src * hkv + g) * (int64_t)D + 8 * c);
    }
  }
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int idx = tid + 256 * j, r = idx / (D / 8), c = idx % (D / 8);
    // K: chunk c of key row r goes to chunk position swz(r, c)
    *reinterpret_cast<u16x8 *>(dst + r * D + 8 * T::template swz<2 * D>(r, c)) = kx[j];
    if (means) *reinterpret_cast<u16x8 *>(&kt[r][8 * c]) = kx[j];
    *reinterpret_cast<u16x8 *>(&vt[r][8 * c]) = vx[j];
  }
  __syncthreads();
  // V^T: row d, stored key slot s <- key vkey(s); chunk c at swz(d, c)
  bool ovf = false;  // a value past fp16's range (flagged in *status)
  for (int idx = tid; idx < D * (kBlk / 8); idx += 256) {
    const int d = idx / (kBlk / 8), c = idx % (kBlk / 8);
    u16x8 val;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t x = vt[T::vkey(8 * c + i)][d];
      val[i] = F16 ? x : bf2h_bits(x);
      ovf |= h16_nonfinite(val[i]);
    }
    *reinterpret_cast<u16x8 *>(dst + T::KE + d * kBlk + 8 * T::template swz<2 * kBlk>(d, c)) = val;
  }
  if (ovf && status) atomicOr(status, kStatusRange);
  if (!means) return;
  const int C = hkv * D, CH = C / 8, P = CH >= 256 ? 1 : 256 / CH;  // P * D <= 2048
#pragma unroll
  for (int kvsel = 0; kvsel < 2; ++kvsel) {
    const uint16_t(*x)[RS] = kvsel ? vt : kt;
    for (int item = tid; item < P * D; item += 256) {
      const int rp = item / D, col = item % D;
      float acc = 0.f;
      for (int r = rp; r < kBlk; r += P) acc += bfbits2f(x[r][col]);
      part[rp * D + col] = acc;
    }
    __syncthreads();
    for (int col = tid; col < D; col += 256) {
      float sum = 0.f;
      for (int rp = 0; rp < P; ++rp) sum += part[rp * D + col];
      (kvsel ? mv : mk)[(int64_t)b * C + g * D + col] = sum * (1.0f / kBlk);
    }
    __syncthreads();
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
                             int split_at, int64_t jump, const int32_t *rows, int32_t *status,
                             float *mk, float *mv, int64_t n_mean) {
  const unsigned n = (unsigned)n_chunks * (unsigned)hkv;
  if (n == 0) return hipSuccess;
  if (v_f16 && mk) return hipErrorInvalidValue;  // means come from bf16 rows only
#define NSA_PACK(D, F)                                                                                  \
  hipLaunchKernelGGL((pack_kv_kernel<D, F>), dim3(n), dim3(256), 0, st, k, v, row0, n_rows, split_at, jump, \
                     hkv, n_chunks, out, rows, status, mk, mv, n_mean)
  if (d == 64) {
    if (v_f16) NSA_PACK(64, true); else NSA_PACK(64, false);
  } else {
    if (v_f16) NSA_PACK(128, true); else NSA_PACK(128, false);
  }
#undef NSA_PACK
  return hipGetLastError();
}

hipError_t launch_pack_kv(const SelParams &p, int d, bool f16, hipStream_t st, float *mk, float *mv,
                          int64_t n_mean) {
  return launch_pack_tiles(p.k, p.v, p.v0, p.n_vis, p.hkv, p.n_frames, p.kv, d, f16, st,
                           0x7fffffff, 0, p.vmap, p.status, mk, mv, n_mean);
}

size_t packed_kv_block_elems(int d) { return (size_t)2 * kBlk * d; }

}  // namespace nsa
