// Token-level branches with a shared key set per query tile: the sliding
// window of vision queries (VideoNSA paper summary page, "Method", branch
// (c)) and dense causal GQA for text queries (same section: text tokens use
// standard GQA).
//
// Layout H: a wave owns 16 queries and up to three of the G query heads of
// one KV group, so each K / V^T fragment read from LDS feeds up to three
// matrix-core ops. Keys and values come from the packed block tiles
// (PackedTile, one 64-key chunk per tile) by direct global->LDS copies, one
// chunk ahead; a single pass with an online softmax forms the output.
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kThreadsH = 256;  // 4 waves x 16 queries
// a row's running max only moves when a new max exceeds it by this many
// log2 units; probabilities stay below 2^slack
constexpr float kSlack = 8.f;

template <int D, int G>
__device__ __forceinline__ void load_q_h(u16x8 (&qf)[G][D / 32], const uint16_t *q, int64_t row0,
                                         bool valid, int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
      qf[h][ds] = valid ? q_frag_global(q + (row0 + h) * D, ds, lane) : zero8();
}

template <int D, int G, bool F16>
__device__ __forceinline__ void qk16(f32x4 (&s)[G], const uint16_t *ks, int kt,
                                     const u16x8 (&qf)[G][D / 32], int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const u16x8 a = pk_k_frag<D>(ks, kt, ds, lane);
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = mfma_qk<F16>(a, qf[h][ds], s[h]);
  }
}

// One staged (K, V^T) chunk for this lane's query row and G heads, online,
// in two halves of 32 keys: scores of the half, the row's running max moved
// lazily (only when a new max exceeds it by kSlack, then the accumulators are
// rescaled), probabilities against that max, then the PV product. Keys
// klo..khi of the chunk (shifted by this lane's 4*(l/16)) are valid for the
// lane's row.
template <int D, int G, bool F16>
__device__ __forceinline__ void online_chunk(const uint16_t *ks, const uint16_t *vt,
                                             const u16x8 (&qf)[G][D / 32], f32x4 (&o)[G][D / 16],
                                             float (&m)[G], float (&l)[G], float sl2, int lane, int klo,
                                             int khi) {
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    f32x4 s[2][G];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kt = 2 * ks2 + kk;
      qk16<D, G, F16>(s[kk], ks, kt, qf, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * kt + i >= klo && 16 * kt + i <= khi;
#pragma unroll
        for (int h = 0; h < G; ++h) s[kk][h][i] = ok ? s[kk][h][i] : -INFINITY;
      }
    }
    u16x8 pf[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h][0];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmax_nn(mx, s[kk][h][i]);
      mx = grp_max(mx) * sl2;  // the row's max over the half (all its lanes)
      if (__builtin_amdgcn_ballot_w64(mx > m[h] + kSlack)) {
        const float mn = fmax_nn(m[h], mx);
        const float alpha = (m[h] == -INFINITY) ? 1.f : exp2f(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[h][dt] = o[h][dt] * alpha;
        m[h] = mn;
      }
      const float nb = (m[h] == -INFINITY) ? 0.f : -m[h];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[kk][h][i] = __builtin_amdgcn_exp2f(fmaf(s[kk][h][i], sl2, nb));
          l[h] += s[kk][h][i];
        }
      pf[h] = pack_p(s[0][h], s[1][h]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u16x8 a = pk_v_frag<D>(vt, dt, ks2, lane);
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][dt] = mfma_f16(a, pf[h], o[h][dt]);
    }
  }
}

// One pass of this lane's query row (G heads) over n_chunks packed chunks
// with the online softmax above. tile_at(c) is chunk c's packed tile;
// key_range(c, lo, hi) gives the keys lo..hi (inclusive, empty if lo > hi)
// of chunk c valid for this lane's row. Returns o normalised and the lse
// (log2 units).
//
// Copies: four separate LDS tiles (64 KB at d = 128, so that two workgroups
// share a CU) hold two (K, V^T) chunk pairs, double-buffered: chunk c+1 is
// in flight while chunk c is used. Each step issues exactly one chunk's
// copies -- past the last chunk they repeat chunk 0 into slots that are
// never read again -- so "chunk c landed" is one straight-line vmcnt wait;
// the slots are separate LDS objects named at compile time, so the compiler
// adds no waits of its own. The slots are the kernel's LDS tiles, passed in
// so that every caller in one kernel shares them.
template <int D, int G, bool F16, class TileAt, class KeyRange>
__device__ __forceinline__ void one_pass(f32x4 (&o)[G][D / 16], float (&lse2)[G],
                                         const u16x8 (&qf)[G][D / 32], float sl2, int n_chunks,
                                         uint16_t (&r0)[PackedTile<D>::KE], uint16_t (&r1)[PackedTile<D>::KE],
                                         uint16_t (&r2)[PackedTile<D>::KE], uint16_t (&r3)[PackedTile<D>::KE],
                                         TileAt tile_at, KeyRange key_range) {
  using T = PackedTile<D>;
  constexpr int KE = T::KE;
  constexpr int PK = KE / 512 / 4;  // copies per wave of one tile
  const int lane = threadIdx.x & 63, g4 = 4 * (lane >> 4);
  const int off = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) * PK * 512);
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[h][dt] = zero4();
  }
#define NSA_KV(DK, DV, C)                                                             \
  {                                                                                   \
    const uint16_t *src_ = tile_at((C) < n_chunks ? (C) : 0);                         \
    dma_pieces<PK>(src_ + off, (DK) + off, lane);                                     \
    dma_pieces<PK>(src_ + KE + off, (DV) + off, lane);                                \
  }
#define NSA_P(CK, CV, NK, NV)                                             \
  {                                                                       \
    wait_vm_c<0>();                                                       \
    bare_barrier();                                                       \
    NSA_KV(NK, NV, c + 1);                                                \
    {                                                                     \
      int lo_, hi_;                                                       \
      key_range(c, lo_, hi_);                                             \
      online_chunk<D, G, F16>(CK, CV, qf, o, m, l, sl2, lane, lo_ - g4, hi_ - g4); \
    }                                                                     \
    if (++c >= n_chunks) break;                                           \
  }
  if (n_chunks > 0) NSA_KV(r0, r1, 0);
  for (int c = 0; c < n_chunks;) {
    NSA_P(r0, r1, r2, r3) NSA_P(r2, r3, r0, r1)
  }
#undef NSA_P
#undef NSA_KV
  wait_vm_c<0>();  // padding copies land before the workgroup's LDS is reused
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float L = grp_sum(l[h]);
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[h][dt] = o[h][dt] * inv;
    lse2[h] = (L > 0.f) ? m[h] + log2f(L) : -INFINITY;
  }
}

// Query heads are split over N workgroups of at most three heads each
// (sizes differing by at most one), so that a wave's accumulators fit half
// the register file: two workgroups share a CU and one's loads and epilogue
// overlap the other's math.
template <int G> struct HeadSplit {
  static constexpr int N = (G + 2) / 3;
  static constexpr int size(int i) { return G / N + (i < G % N ? 1 : 0); }
  static constexpr int first(int i) { return i == 0 ? 0 : first(i - 1) + size(i - 1); }
};

// Workgroups are handed to the eight XCDs round-robin by index, and each XCD
// has its own L2. The launch is padded to a multiple of eight and index i is
// mapped to the logical item (i % 8) * per + i / 8, so each XCD works through
// one contiguous range of items; items that read the same key tiles are made
// adjacent, so those tiles come from the XCD's L2 after the first read.
// Returns -1 for the padding.
__device__ __forceinline__ int xcd_item(int i, int n_items) {
  const int per = (n_items + 7) / 8;
  const int item = (i % 8) * per + i / 8;
  return item < n_items ? item : -1;
}
__host__ inline unsigned xcd_grid(unsigned n_items) { return (n_items + 7) / 8 * 8; }

// ----------------------------------------------------------- sliding window
// A 64-query tile (vision frame f) needs keys [t0 - w + 1, t0 + 63], i.e.
// the packed blocks from (t0 - w + 1) / 64 to f.
template <int D> struct Ring4 {
  uint16_t (&r0)[PackedTile<D>::KE], (&r1)[PackedTile<D>::KE], (&r2)[PackedTile<D>::KE], (&r3)[PackedTile<D>::KE];
};

template <int D, int G, bool F16, int HW, int H0>
__device__ __forceinline__ void swa_body(const SwaParams &p, int g, int f, Ring4<D> rg) {
  using T = PackedTile<D>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4;
  const int t0 = f * kBlk;
  const int t = t0 + wv * 16 + (lane & 15);
  const bool tvalid = t < p.n_vis;
  const int b_lo = max(0, t0 - p.window + 1) / kBlk;
  const int wnd = p.window;

  u16x8 qf[HW][D / 32];
  const int64_t qrow = row_pos(p.vmap, p.v0, tvalid ? t : 0) * p.hq + (int64_t)g * G + H0;
  load_q_h<D, HW>(qf, p.q, qrow, tvalid, lane);
  f32x4 o[HW][D / 16];
  float lse2[HW];
  const uint16_t *tiles = p.kv + ((int64_t)g * p.n_tiles + b_lo) * (T::KE + T::VE);
  one_pass<D, HW, F16>(o, lse2, qf, p.sl2, f - b_lo + 1, rg.r0, rg.r1, rg.r2, rg.r3,
                          [&](int c) { return tiles + (int64_t)c * (T::KE + T::VE); },
                          [&](int c, int &lo, int &hi) {
                            const int key0 = (b_lo + c) * kBlk;  // keys t-w+1 .. t
                            lo = t - wnd + 1 - key0;
                            hi = tvalid ? t - key0 : -1;
                          });
  if (tvalid) {  // sigmoid(g_swa) * o_swa as the fp16 part 1 of the row's output slots
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float gate = sigmoidf_(p.gates[(qrow + h) * 3 + 2]);
      float *slot = p.out + (qrow + h) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) store_partial4<D>(slot, 1, 16 * dt + 4 * grp, o[h][dt] * gate);
    }
  }
}

template <int D, int G, bool F16>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void swa_attn_kernel(SwaParams p) {
  using S = HeadSplit<G>;
  constexpr int KE = PackedTile<D>::KE;
  __shared__ __attribute__((aligned(16))) uint16_t r0[KE], r1[KE], r2[KE], r3[KE];
  const Ring4<D> rg{r0, r1, r2, r3};
  // item order: head part fastest, then frame, then KV group, so one XCD
  // takes consecutive frames of one group (neighbouring frames' windows
  // share all but one key tile)
  const int item = xcd_item(blockIdx.x, p.n_tiles * p.hkv * S::N);
  if (item < 0) return;
  const int half = item % S::N, rest = item / S::N;
  const int f = rest % p.n_tiles;
  const int g = rest / p.n_tiles;
  if (half == 0) swa_body<D, G, F16, S::size(0), 0>(p, g, f, rg);
  else if constexpr (S::N > 1) {
    if (half == 1) swa_body<D, G, F16, S::size(1), S::first(1)>(p, g, f, rg);
    else if constexpr (S::N > 2) swa_body<D, G, F16, S::size(2), S::first(2)>(p, g, f, rg);
  }
}

// --------------------------------------------------------------- text rows
// Position of text row r: from the map when the vision tokens lie in several
// runs, else the rows before the one vision run [v0, v1), then those after.
__device__ __forceinline__ int64_t text_pos(const TextParams &p, int r) {
  return p.tmap ? (int64_t)p.tmap[r] : r < p.v0 ? (int64_t)r : p.v1 + (r - p.v0);
}

// One (64-query text tile, KV group, key split, head part) per workgroup.
// The keys of the whole sequence are the packed vision chunks followed by
// the packed text chunks; split sp takes chunks [sp * cps, (sp + 1) * cps).
// Writes the split's normalised output and lse for the merge kernel.
template <int D, int G, bool F16, int HW, int H0>
__device__ __forceinline__ void text_body(const TextParams &p, int sp, int g, int tile, Ring4<D> rg) {
  using T = PackedTile<D>;
  constexpr int SE = T::KE + T::VE;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4;
  const int r = tile * kBlk + wv * 16 + (lane & 15);
  const bool rvalid = r < p.n_text;
  const int64_t pos = rvalid ? text_pos(p, r) : -1;
  const int nvc = p.n_vchunks, nch = p.n_vchunks + p.n_tchunks;
  const int cb = sp * p.chunks_per_split, ce = min(cb + p.chunks_per_split, nch);
  // vision keys before the query: a prefix of the vision rows
  const int64_t n_vb = !rvalid ? 0 : p.tnvb ? (int64_t)p.tnvb[r] : pos < p.v0 ? 0 : p.v1 - p.v0;

  u16x8 qf[HW][D / 32];
  const int64_t qrow = (rvalid ? pos : 0) * p.hq + (int64_t)g * G + H0;
  load_q_h<D, HW>(qf, p.q, qrow, rvalid, lane);
  f32x4 o[HW][D / 16];
  float lse2[HW];
  const uint16_t *vis = p.kv_vis + (int64_t)g * p.n_vchunks * SE;
  const uint16_t *txt = p.kv_txt + (int64_t)g * p.n_tchunks * SE;
  one_pass<D, HW, F16>(o, lse2, qf, p.sl2, max(0, ce - cb), rg.r0, rg.r1, rg.r2, rg.r3,
                          [&](int c) {
                            const int cc = cb + c;
                            return cc < nvc ? vis + (int64_t)cc * SE : txt + (int64_t)(cc - nvc) * SE;
                          },
                          [&](int c, int &lo, int &hi) {
                            const int cc = cb + c;
                            lo = 0;
                            if (cc < nvc) {  // vision-local keys j < n_vb
                              hi = (int)n_vb - 1 - cc * kBlk;
                            } else {  // text-local keys j: positions increase with j, so j <= r
                              hi = (rvalid ? r : -1) - (cc - nvc) * kBlk;
                            }
                          });
  if (rvalid) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const int64_t pr = ((int64_t)sp * p.n_text + r) * p.hq + g * G + H0 + h;
      if (grp == 0) p.part_ml[pr] = make_float2(lse2[h], 0.f);
      float *dst = p.part_o + pr * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = o[h][dt];
    }
  }
}

template <int D, int G, bool F16>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void text_attn_kernel(TextParams p) {
  using S = HeadSplit<G>;
  constexpr int KE = PackedTile<D>::KE;
  __shared__ __attribute__((aligned(16))) uint16_t r0[KE], r1[KE], r2[KE], r3[KE];
  const Ring4<D> rg{r0, r1, r2, r3};
  // item order: head part fastest, then query tile, then key split, then KV
  // group, so the workgroups reading one split's key tiles run together on
  // one XCD
  const int item = xcd_item(blockIdx.x, p.n_tiles * p.hkv * p.n_split * S::N);
  if (item < 0) return;
  const int half = item % S::N;
  const int rest0 = item / S::N;
  const int tile = rest0 % p.n_tiles;
  const int rest = rest0 / p.n_tiles;
  const int sp = rest % p.n_split;
  const int g = rest / p.n_split;
  if (half == 0) text_body<D, G, F16, S::size(0), 0>(p, sp, g, tile, rg);
  else if constexpr (S::N > 1) {
    if (half == 1) text_body<D, G, F16, S::size(1), S::first(1)>(p, sp, g, tile, rg);
    else if constexpr (S::N > 2) text_body<D, G, F16, S::size(2), S::first(2)>(p, sp, g, tile, rg);
  }
}

// Combines the key splits of every (text query, head): each split carries a
// normalised output and its lse (log2 units); weights are exp2(lse_s - LSE).
template <int D>
__global__ __launch_bounds__(D) void text_merge_kernel(TextParams p) {
  const int r = blockIdx.x / p.hq, h = blockIdx.x % p.hq, d = threadIdx.x;
  // the splits' loads are independent: unrolled, many are in flight at once
  float M = -INFINITY;
#pragma unroll 16
  for (int sp = 0; sp < p.n_split; ++sp)
    M = fmax_nn(M, p.part_ml[((int64_t)sp * p.n_text + r) * p.hq + h].x);
  float acc = 0.f, L = 0.f;
#pragma unroll 16
  for (int sp = 0; sp < p.n_split; ++sp) {
    const int64_t pr = ((int64_t)sp * p.n_text + r) * p.hq + h;
    const float lse = p.part_ml[pr].x;
    const float w = (lse == -INFINITY) ? 0.f : exp2f(lse - M);  // an empty split weighs 0
    L += w;
    acc += w * p.part_o[pr * D + d];
  }
  p.out[(text_pos(p, r) * p.hq + h) * D + d] = acc / L;
}

// ------------------------------------------------------- dense causal GQA
// Every token attends to every earlier token and itself (the Dense-NSA mode
// of the VideoNSA paper summary page, "Key claims" and "Results": the
// sparse-trained weights run under full attention). One (64-query tile, KV
// group, head part) per workgroup over the packed chunks 0 .. tile; only the
// last chunk is masked. Work per tile grows with the tile index, so tiles go
// heaviest first (longest-processing-time order as slots free up); the head
// parts of one (tile, group) sit eight ids apart, i.e. on one XCD at about
// the same time, and share its L2 for the key tiles.
template <int D, int G, bool F16, int HW, int H0>
__device__ __forceinline__ void dense_body(const DenseParams &p, int g, int tile, Ring4<D> rg) {
  using T = PackedTile<D>;
  constexpr int SE = T::KE + T::VE;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4;
  const int64_t r = (int64_t)tile * kBlk + wv * 16 + (lane & 15);
  const bool rvalid = r < p.n;
  u16x8 qf[HW][D / 32];
  const int64_t qrow = (rvalid ? r : 0) * p.hq + (int64_t)g * G + H0;
  load_q_h<D, HW>(qf, p.q, qrow, rvalid, lane);
  f32x4 o[HW][D / 16];
  float lse2[HW];
  const uint16_t *kv = p.kv + (int64_t)g * p.n_tiles * SE;
  const int rl = rvalid ? (int)(r - (int64_t)tile * kBlk) : -1;  // row within the last chunk
  one_pass<D, HW, F16>(o, lse2, qf, p.sl2, tile + 1, rg.r0, rg.r1, rg.r2, rg.r3,
                       [&](int c) { return kv + (int64_t)c * SE; },
                       [&](int c, int &lo, int &hi) {
                         lo = 0;
                         hi = !rvalid ? -1 : c < tile ? kBlk - 1 : rl;
                       });
  if (rvalid) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      if (p.lse && grp == 0) p.lse[qrow + h] = lse2[h] * 0.69314718055994531f;
      float *dst = p.out + (qrow + h) * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = o[h][dt];
    }
  }
}

template <int D, int G, bool F16>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_attn_kernel(DenseParams p) {
  using S = HeadSplit<G>;
  constexpr int KE = PackedTile<D>::KE;
  __shared__ __attribute__((aligned(16))) uint16_t r0[KE], r1[KE], r2[KE], r3[KE];
  const Ring4<D> rg{r0, r1, r2, r3};
  const int i = blockIdx.x;
  const int half = (i >> 3) % S::N;
  const int u = (i / (8 * S::N)) * 8 + (i & 7);  // (tile, group), heaviest first
  if (u >= p.n_tiles * p.hkv) return;
  const int tile = p.n_tiles - 1 - u / p.hkv;
  const int g = u % p.hkv;
  if (half == 0) dense_body<D, G, F16, S::size(0), 0>(p, g, tile, rg);
  else if constexpr (S::N > 1) {
    if (half == 1) dense_body<D, G, F16, S::size(1), S::first(1)>(p, g, tile, rg);
    else if constexpr (S::N > 2) dense_body<D, G, F16, S::size(2), S::first(2)>(p, g, tile, rg);
  }
}

// ------------------------------------------------------------- launchers
template <int D, int G, bool F16>
hipError_t run_swa(const SwaParams &p, hipStream_t st) {
  const unsigned n = (unsigned)p.n_tiles * (unsigned)p.hkv * HeadSplit<G>::N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((swa_attn_kernel<D, G, F16>), dim3(xcd_grid(n)), dim3(kThreadsH), 0, st, p);
  return hipGetLastError();
}

template <int D, int G, bool F16>
hipError_t run_text(const TextParams &p, hipStream_t st) {
  const unsigned n = (unsigned)p.n_tiles * (unsigned)p.hkv * (unsigned)p.n_split * HeadSplit<G>::N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((text_attn_kernel<D, G, F16>), dim3(xcd_grid(n)), dim3(kThreadsH), 0, st, p);
  return hipGetLastError();
}

template <int D, int G, bool F16>
hipError_t run_dense(const DenseParams &p, hipStream_t st) {
  const unsigned u = (unsigned)p.n_tiles * (unsigned)p.hkv;
  if (u == 0) return hipSuccess;
  const unsigned n = (u + 7) / 8 * 8 * HeadSplit<G>::N;
  hipLaunchKernelGGL((dense_attn_kernel<D, G, F16>), dim3(n), dim3(kThreadsH), 0, st, p);
  return hipGetLastError();
}

#define NSA_SWITCH_G(FN, VF, ...)                               \
  if (d == 64) {                                                \
    switch (G) {                                                \
      case 1: return FN<64, 1, VF>(__VA_ARGS__);                \
      case 2: return FN<64, 2, VF>(__VA_ARGS__);                \
      case 3: return FN<64, 3, VF>(__VA_ARGS__);                \
      case 4: return FN<64, 4, VF>(__VA_ARGS__);                \
      case 5: return FN<64, 5, VF>(__VA_ARGS__);                \
      case 6: return FN<64, 6, VF>(__VA_ARGS__);                \
      case 7: return FN<64, 7, VF>(__VA_ARGS__);                \
      case 8: return FN<64, 8, VF>(__VA_ARGS__);                \
    }                                                           \
  } else if (d == 128) {                                        \
    switch (G) {                                                \
      case 1: return FN<128, 1, VF>(__VA_ARGS__);               \
      case 2: return FN<128, 2, VF>(__VA_ARGS__);               \
      case 3: return FN<128, 3, VF>(__VA_ARGS__);               \
      case 4: return FN<128, 4, VF>(__VA_ARGS__);               \
      case 5: return FN<128, 5, VF>(__VA_ARGS__);               \
      case 6: return FN<128, 6, VF>(__VA_ARGS__);               \
      case 7: return FN<128, 7, VF>(__VA_ARGS__);               \
    }                                                           \
  }                                                             \
  return hipErrorInvalidValue;

}  // namespace

hipError_t launch_swa_attn(const SwaParams &p, int d, int G, bool f16, hipStream_t st) {
  if (f16) { NSA_SWITCH_G(run_swa, true, p, st) }
  NSA_SWITCH_G(run_swa, false, p, st)
}
hipError_t launch_text_merge(const TextParams &p, int d, hipStream_t st) {
  if (p.n_text == 0) return hipSuccess;
  if (d == 64) hipLaunchKernelGGL((text_merge_kernel<64>), dim3((unsigned)(p.n_text * p.hq)), dim3(64), 0, st, p);
  else hipLaunchKernelGGL((text_merge_kernel<128>), dim3((unsigned)(p.n_text * p.hq)), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_text_attn(const TextParams &p, int d, int G, bool f16, hipStream_t st) {
  if (f16) { NSA_SWITCH_G(run_text, true, p, st) }
  NSA_SWITCH_G(run_text, false, p, st)
}

hipError_t launch_dense_attn(const DenseParams &p, int d, int G, bool f16, hipStream_t st) {
  if (f16) { NSA_SWITCH_G(run_dense, true, p, st) }
  NSA_SWITCH_G(run_dense, false, p, st)
}
}  // namespace nsa
