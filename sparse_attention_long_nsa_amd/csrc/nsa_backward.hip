// Backward pass of the layer for training (model card, "Training Details";
// paper summary, "Method": the model is trained end to end through the NSA
// branches and gates). The block selection is a discrete choice with no
// gradient, so the forward's selected blocks are an input; gradients flow to
// q, k, v (all three branches and the text rows), the gate logits and both
// compression maps.
//
// Every attention branch is differentiated the same way, on the matrix
// cores (fp16 operands, fp32 accumulation), with each gradient element
// written by exactly one thread and no atomics, so results are bitwise
// repeatable:
//   bwd_pool      block means and compressed keys / values (fp32, plus fp16
//                 copies for the matrix cores)
//   bwd_pack      per (64-key tile, KV group) two fp16 sections, K rows
//                 and V rows (16-byte chunks swizzled per row), for the
//                 vision blocks, for every position (text queries) and for
//                 the compressed keys
//   bwd_selmask.. the tokens that chose each (group, block), ascending: a
//                 bitmask over tokens, its row counts, their prefix sum and
//                 the decoded lists
//   bwd_q         query side, one wave per (tile of 16/G tokens, KV group),
//                 eight consecutive tiles per workgroup sharing each key tile
//                 staged once in LDS (window, compression: walked in
//                 lockstep; selection: a three-slot ring that each wave walks
//                 at its own pace over the tiles its tokens chose, refilled
//                 by idle waves): per branch, pass 1 recomputes the
//                 branch's log-sum-exp and output o (online softmax), giving
//                 D = dout . o and the gate gradient; pass 2 forms
//                 dS = sigma P (dP - D) and dq^T += K^T dS^T; V^T and K^T
//                 come out of the staged rows through the transposing LDS
//                 read; dq is written once after all branches (text rows:
//                 split over key tiles)
//   bwd_kv        key side, one workgroup per (64-key tile, KV group), a
//                 wave per 16 keys: walks every query row that attends the
//                 tile (window range, selection list, text rows) 32 rows at
//                 a time; dV^T += dO^T P and dK^T += Q^T dS with the rows'
//                 Q^T and dO^T read from their row-major LDS staging by the
//                 transposing LDS read; dk, dv written once
//   bwd_kvc /     the same for the compressed keys over chunks of 2,048
//   bwd_creduce   query tokens, the chunks' partial sums then added in order
//   bwd_cmp_w /   dW = sum over blocks of dK_cmp x mean^T, and each block's
//   bwd_cmp_tok   W^T dK_cmp / 64 added to its 64 tokens' dk (dv likewise)
#include <type_traits>

#include "nsa_kernels.h"
#include "nsa_index.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kSentinel = 0x7fffffff;
constexpr int kChunkTok = 2048;  // query tokens per compressed-key partial

// Whether any of eight fp16 values overflowed the fp16 range on conversion.
__device__ __forceinline__ bool any_nonfinite8(u16x8 x) {
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) bad |= h16_nonfinite(x[i]);
  return bad;
}

// four 16-bit values, and the LDS pointer type the transposing read takes
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D>
struct BwdTile {
  static constexpr int SEC = kBlk * D;  // elements per section
  static constexpr int E = 2 * SEC;     // sections: K rows, V rows
};

__global__ void bwd_fill_kernel(uint32_t *a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a[i] = 0u;
}

// One workgroup of D threads per (block, KV group): means of the block's 64
// vision rows and their image under W (y = W x), for keys and values.
template <int D>
__global__ __launch_bounds__(D) void bwd_pool_kernel(BwdParams p) {
  __shared__ float xm[2][D];
  const int b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv, i = threadIdx.x;
  const int64_t r0 = p.v0 + (int64_t)b * kBlk;
  float sk = 0.f, sv = 0.f;
  for (int r = 0; r < kBlk; ++r) {
    const int64_t o = ((r0 + r) * p.hkv + g) * D + i;
    sk += bfbits2f(p.k[o]);
    sv += bfbits2f(p.v[o]);
  }
  sk *= 1.f / kBlk;
  sv *= 1.f / kBlk;
  xm[0][i] = sk;
  xm[1][i] = sv;
  const int64_t ob = ((int64_t)b * p.hkv + g) * D + i;
  p.kbar[ob] = sk;
  p.vbar[ob] = sv;
  __syncthreads();
  float yk = 0.f, yv = 0.f;
  for (int j = 0; j < D; ++j) {
    yk = fmaf(bfbits2f(p.wk[i * D + j]), xm[0][j], yk);
    yv = fmaf(bfbits2f(p.wv[i * D + j]), xm[1][j], yv);
  }
  p.kc[ob] = yk;
  p.vc[ob] = yv;
  p.kc16[ob] = f2h_bits(yk);
  p.vc16[ob] = f2h_bits(yv);
  if (h16_nonfinite(f2h_bits(yk)) || h16_nonfinite(f2h_bits(yv))) atomicOr(p.status, kStatusRange);
}

// Packs rows row0 .. row0 + n_rows - 1 of a [rows][Hkv][D] key and value
// array (bf16, converted, or fp16) into backward tiles: tile i holds rows
// row0 + 64 i .. +63 (zero past n_rows). One workgroup per (tile, group).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_pack_kernel(const uint16_t *ksrc, const uint16_t *vsrc, int64_t row0,
                                                       int64_t n_rows, int hkv, int n_tiles, uint16_t *dst,
                                                       int32_t *status) {
  constexpr int SEC = BwdTile<D>::SEC, CH = D / 8;
  const int tile = blockIdx.x % n_tiles, g = blockIdx.x / n_tiles;
  uint16_t *out = dst + ((int64_t)g * n_tiles + tile) * BwdTile<D>::E;
  for (int idx = threadIdx.x; idx < 2 * kBlk * CH; idx += 256) {
    const int w = idx / (kBlk * CH), r = (idx / CH) % kBlk, c = idx % CH;
    const int64_t row = (int64_t)tile * kBlk + r;
    u16x8 x = zero8();
    if (row < n_rows) {
      x = *reinterpret_cast<const u16x8 *>((w ? vsrc : ksrc) + ((row0 + row) * hkv + g) * D + 8 * c);
      if constexpr (BF16) {
        x = bf2h8(x);
        if (any_nonfinite8(x)) atomicOr(status, kStatusRange);
      }
    }
    *reinterpret_cast<u16x8 *>(out + w * SEC + r * D + 8 * PackedTile<D>::template swz<2 * D>(r, c)) = x;
  }
}

// ------------------------------------------------- who chose which block
// bit t of selmask[g][b] = vision token t has block b in its list (entries
// outside 0 .. t / 64 are ignored, as on the query side).
__global__ void bwd_selmask_kernel(BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, g, e)
  if (i >= p.n_vis * p.hkv * p.topk) return;
  const int t = (int)(i / ((int64_t)p.hkv * p.topk));
  const int g = (int)((i / p.topk) % p.hkv);
  const int32_t b = p.sel[i];
  if (!sel_entry_valid(b, t)) return;
  atomicOr(&p.selmask[((int64_t)g * p.n_vtile + b) * p.mask_words + (t >> 5)], 1u << (t & 31));
}

// One wave per (group, block): number of tokens that chose it.
__global__ __launch_bounds__(64) void bwd_selcount_kernel(BwdParams p) {
  const int gb = blockIdx.x, lane = threadIdx.x;
  const uint32_t *row = p.selmask + (int64_t)gb * p.mask_words;
  int c = 0;
  for (int w = lane; w < p.mask_words; w += 64) c += __popc(row[w]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) p.selcnt[gb] = c;
}

// Exclusive prefix sum of the counts (one workgroup): seloff[i] = sum of
// counts before i, seloff[n] = the total.
__global__ __launch_bounds__(256) void bwd_selscan_kernel(BwdParams p, int n) {
  __shared__ int part[256];
  const int tid = threadIdx.x, per = (n + 255) / 256;
  const int a = min(n, tid * per), b = min(n, a + per);
  int s = 0;
  for (int i = a; i < b; ++i) s += p.selcnt[i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    p.seloff[n] = run;
  }
  __syncthreads();
  int run = part[tid];
  for (int i = a; i < b; ++i) {
    p.seloff[i] = run;
    run += p.selcnt[i];
  }
}

// One wave per (group, block): writes the tokens of its bitmask row, in
// ascending order, at its offset.
__global__ __launch_bounds__(64) void bwd_selfill_kernel(BwdParams p) {
  const int gb = blockIdx.x, lane = threadIdx.x;
  const uint32_t *row = p.selmask + (int64_t)gb * p.mask_words;
  int base = p.seloff[gb];
  for (int w0 = 0; w0 < p.mask_words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t bits = w < p.mask_words ? row[w] : 0u;
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int at = base + incl - c;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      p.selrows[at++] = 32 * w + bit;
      bits &= bits - 1u;
    }
    base += __shfl(incl, 63);
  }
}

// ------------------------------------------------------------ query side
constexpr int kQWaves = 8;        // query tiles (one per wave) per workgroup
constexpr int kMaxVTile = 8192;   // vision blocks (the prefill limit)
constexpr int kMaxTopk = 64;

// Scores of one tile transposed: s[kt] = K_kt Q^T (16 keys x 16 rows each)
// from a section of K rows (or of V rows, for dP^T = V dO^T).
template <int D>
__device__ __forceinline__ void tile_scores(const uint16_t *sec, const u16x8 (&b)[D / 32], f32x4 (&s)[4],
                                            int lane) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) s[kt] = zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = mfma_f16(pk_k_frag<D>(sec, kt, ds, lane), b[ds], s[kt]);
}

// A operand (16 dims x 32 keys) of key half kh from a staged section of K
// or V rows (row-major, 16-byte chunks swizzled per row), through the
// transposing LDS read: lane l gets dim 16 dt + l % 16 at keys
// 32 kh + 4 (l / 16) + j (elements 0-3) and 32 kh + 16 + 4 (l / 16) + j
// (elements 4-7), the key-slot order of the P and dS operands. Within each
// 16-lane group the read hands lane i element j of the 8 bytes that lane
// i / 4 + 4 j addressed; lane s addresses keys 4 (l / 16) + s / 4 (+ 16),
// dims 16 dt + 4 (s % 4) .. + 3.
template <int D>
__device__ __forceinline__ u16x8 sec_tr_frag(const uint16_t *sec, int dt, int kh, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int r0 = 32 * kh + 4 * g + (s >> 2), r1 = r0 + 16;
  const int d = 16 * dt + 4 * (s & 3), c = d >> 3, h = d & 7;  // chunk of the four dims, and 0 or 4 in it
  const uint16_t *p0 = sec + r0 * D + 8 * PackedTile<D>::template swz<2 * D>(r0, c) + h;
  const uint16_t *p1 = sec + r1 * D + 8 * PackedTile<D>::template swz<2 * D>(r1, c) + h;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p1);
  return u16x8{(uint16_t)a[0], (uint16_t)a[1], (uint16_t)a[2], (uint16_t)a[3],
               (uint16_t)b[0], (uint16_t)b[1], (uint16_t)b[2], (uint16_t)b[3]};
}

// Pass 1 over one tile (sections K rows and V rows): online max and sum of the
// row's exponentials (log2 domain) and O^T += V^T P^T. valid(kt, i) says
// whether the row sees key 16 kt + 4 (lane / 16) + i of the tile.
template <int D, class Valid>
__device__ __forceinline__ void q_pass1(const uint16_t *kp, const uint16_t *vp, const u16x8 (&qf)[D / 32],
                                        f32x4 (&oa)[D / 16], float &m, float &l, float sl2, Valid valid, int lane) {
  f32x4 s[4];
  tile_scores<D>(kp, qf, s, lane);
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = valid(kt, i) ? s[kt][i] * sl2 : -INFINITY;
      s[kt][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = grp_max(mx);
  const float mn = fmaxf(m, mx);
  const bool live = mn != -INFINITY;
  const float alpha = live ? exp2f(m - mn) : 1.f;
  l *= alpha;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oa[dt] = oa[dt] * alpha;
  float ls = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = live ? __builtin_amdgcn_exp2f(s[kt][i] - mn) : 0.f;
      s[kt][i] = pv;
      ls += pv;
    }
  l += ls;
  m = mn;
  const u16x8 pp[2] = {pack_p(s[0], s[1]), pack_p(s[2], s[3])};
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oa[dt] = mfma_f16(sec_tr_frag<D>(vp, dt, kh, lane), pp[kh], oa[dt]);
}

// Pass 2 over one tile (sections K rows and V rows): P from the row's
// log-sum-exp, dP^T = V dO^T, dS = sig P (dP - dd), dq^T += K^T dS^T.
template <int D, class Valid>
__device__ __forceinline__ void q_pass2(const uint16_t *kp, const uint16_t *vp,
                                        const u16x8 (&qf)[D / 32], const u16x8 (&of)[D / 32], f32x4 (&dqa)[D / 16],
                                        float lse2, float dd, float sig, float sl2, Valid valid, int lane) {
  f32x4 s[4], dp[4];
  tile_scores<D>(kp, qf, s, lane);
  tile_scores<D>(vp, of, dp, lane);
  const bool has = lse2 != -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = (has && valid(kt, i)) ? __builtin_amdgcn_exp2f(fmaf(s[kt][i], sl2, -lse2)) : 0.f;
      s[kt][i] = sig * pv * (dp[kt][i] - dd);
    }
  const u16x8 pd[2] = {pack_p(s[0], s[1]), pack_p(s[2], s[3])};
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) dqa[dt] = mfma_f16(sec_tr_frag<D>(kp, dt, kh, lane), pd[kh], dqa[dt]);
}

// Query rows of one wave: TP tokens x G heads (+ padding rows) of one KV
// group; lane l owns row l % 16. TXT: text rows (index u among the text
// tokens), else vision rows.
template <int D, int G, bool TXT>
struct QRows {
  static constexpr int TP = 16 / G;
  int tau, hh, grp, tok, hq;
  bool rv;
  int64_t pos, qrow;
  __device__ QRows(const BwdParams &p, int qt, int g, int lane) {
    const int r16 = lane & 15;
    tau = r16 / G;
    hh = r16 % G;
    grp = lane >> 4;
    const int n_tok = TXT ? (int)(p.n - p.n_vis) : (int)p.n_vis;
    tok = qt * TP + tau;
    rv = tau < TP && tok < n_tok;
    const int tc = rv ? tok : 0;
    pos = TXT ? (tc < p.v0 ? (int64_t)tc : (int64_t)tc + p.n_vis) : p.v0 + tc;
    hq = g * G + hh;
    qrow = pos * p.hq + hq;
  }
};

// The query operands of a wave: Q^T and dO^T fragments (B operands, fp16;
// a value past the fp16 range sets the status word).
template <int D>
__device__ __forceinline__ void q_operands(const BwdParams &p, bool rv, int64_t qrow, u16x8 (&qf)[D / 32],
                                           u16x8 (&of)[D / 32], int lane) {
  bool bad = false;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    qf[ds] = rv ? bf2h8(q_frag_global(p.q + qrow * D, ds, lane)) : zero8();
    u16x8 o = zero8();
    if (rv) {
      const float *src = p.dout + qrow * D + 32 * ds + 8 * (lane >> 4);
      o = pack_p(*reinterpret_cast<const f32x4 *>(src), *reinterpret_cast<const f32x4 *>(src + 4));
    }
    of[ds] = o;
    bad |= any_nonfinite8(qf[ds]) || any_nonfinite8(o);
  }
  if (bad) atomicOr(p.status, kStatusRange);
}

// The workgroup walks n tiles in lockstep (n and tile_of(i), the global
// base of tile i, are the same for every wave): each step copies the next
// tile's two sections (K rows, V rows) into the other LDS buffer by direct
// global->LDS loads, the copies split over the waves, while every wave runs
// body(i, staged sections) on the current tile; then each wave waits for its
// own copies and the workgroup meets at a barrier. The two buffers are
// separate LDS objects and each step names its buffers at compile time, so
// the reads of one need not wait for the copies still landing in the other.
template <int D, int PASS, class TileOf, class Body>
__device__ __forceinline__ void lockstep(int n, TileOf tile_of, uint16_t (&l0)[2 * BwdTile<D>::SEC],
                                         uint16_t (&l1)[2 * BwdTile<D>::SEC], Body body, int wv, int lane) {
  constexpr int SEC = BwdTile<D>::SEC, NSEC = 2, PPS = SEC / 512, PPW = NSEC * PPS / kQWaves;
  static_assert((NSEC * PPS) % kQWaves == 0, "copies split evenly over the waves");
  auto copy = [&](const uint16_t *src, uint16_t *dst) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int pc = wv * PPW + j, sl = pc / PPS, off = pc % PPS;
      __builtin_amdgcn_global_load_lds(src + sl * SEC + off * 512 + lane * 8,
                                       (lds_void *)(dst + sl * SEC + off * 512), 16, 0, 0);
    }
  };
  if (n <= 0) return;
  copy(tile_of(0), l0);
  wait_vm_c<0>();
  bare_barrier();
  for (int i = 0; i < n;) {
    if (i + 1 < n) copy(tile_of(i + 1), l1);
    body(i, static_cast<const uint16_t *>(l0));
    wait_vm_c<0>();
    bare_barrier();
    if (++i >= n) break;
    if (i + 1 < n) copy(tile_of(i + 1), l0);
    body(i, static_cast<const uint16_t *>(l1));
    wait_vm_c<0>();
    bare_barrier();
    ++i;
  }
}

// One branch for the wave's rows: pass 1 (log-sum-exp, o, then D = dout . o,
// the statistics for the key side and the gate gradient), pass 2 (dq).
// walk(pass tag, f) calls f(K rows, V rows, valid) for the tiles the wave
// needs, in the same order in both passes.
template <int D, class Walk>
__device__ __forceinline__ void q_branch(const BwdParams &p, Walk walk, const u16x8 (&qf)[D / 32],
                                         const u16x8 (&of)[D / 32], f32x4 (&dqa)[D / 16], bool rv,
                                         int64_t qrow, float sig, float sl2, float *stat, float *dgate,
                                         int lane) {
  constexpr int DT = D / 16;
  f32x4 oa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oa[dt] = zero4();
  float m = -INFINITY, l = 0.f;
  walk(std::integral_constant<int, 1>(), [&](const uint16_t *s0, const uint16_t *s1, auto valid) {
    q_pass1<D>(s0, s1, qf, oa, m, l, sl2, valid, lane);
  });
  const float L = grp_sum(l);
  const bool has = rv && L > 0.f;
  const float lse2 = has ? m + __log2f(L) : -INFINITY;
  const int grp = lane >> 4;
  // D from dout rounded to fp16 as in the products that form dP, so that
  // dP - D cancels exactly where the row's probability mass sits on one key
  float part = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const f32x4 dv = rv ? *reinterpret_cast<const f32x4 *>(p.dout + qrow * D + 16 * dt + 4 * grp) : zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) part = fmaf(h16_to_f32(f2h_bits(dv[i])), oa[dt][i], part);
  }
  part = grp_sum(part);
  const float dd = has ? part / L : 0.f;
  if (rv && grp == 0) {
    stat[0] = lse2;
    stat[1] = dd;
    if (dgate) *dgate = sig * (1.f - sig) * dd;
  }
  walk(std::integral_constant<int, 2>(), [&](const uint16_t *s0, const uint16_t *s1, auto valid) {
    q_pass2<D>(s0, s1, qf, of, dqa, lse2, dd, sig, sl2, valid, lane);
  });
}

// Vision rows: workgroup = kQWaves consecutive query tiles of one KV group;
// the three branches' key tiles are staged once for all its waves.
template <int D, int G>
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(2))) void bwd_q_kernel(BwdParams p,
                                                                                                    int n_qt) {
  using R = QRows<D, G, false>;
  constexpr int TP = R::TP, DT = D / 16, SEC = BwdTile<D>::SEC, E = BwdTile<D>::E, TW = TP * kQWaves;
  __shared__ __attribute__((aligned(16))) uint16_t lds0[2 * SEC], lds1[2 * SEC];  // the two step buffers
  __shared__ __attribute__((aligned(16))) uint16_t lds2[2 * SEC];  // third ring slot (selection)
  __shared__ uint32_t ubits[kMaxVTile / 32];   // union of the workgroup's selected blocks
  __shared__ int16_t wpre[kMaxVTile / 32];     // union entries before each bitmask word
  __shared__ uint16_t ulist[TW * kMaxTopk];    // the union, ascending
  __shared__ int n_union;
  __shared__ int rpass[kQWaves], rready[3], rnext;  // selection ring: see ring_walk
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // workgroups go to the eight XCDs round-robin: give each XCD one
  // contiguous run of query tiles (neighbours share key tiles in its L2)
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int wg = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int n_grp = (n_qt + kQWaves - 1) / kQWaves;
  if (wg >= n_grp * p.hkv) return;  // the whole workgroup
  const int g = wg / n_grp, qg = wg % n_grp, qt = qg * kQWaves + wv;
  const R r(p, qt, g, lane);
  const float sl2 = p.scale * kLog2e;
  const int n_tok = (int)p.n_vis;
  const int wt_first = qg * TW, wt_last = min(qg * TW + TW, n_tok) - 1;  // the workgroup's tokens
  const int t_first = qt * TP, t_last = min(qt * TP + TP, n_tok) - 1;    // the wave's (t_last < t_first: none)
  const int grp = r.grp, tok = r.tok;
  u16x8 qf[D / 32], of[D / 32];
  q_operands<D>(p, r.rv, r.qrow, qf, of, lane);
  f32x4 dqa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqa[dt] = zero4();
  float *stat = p.vstat + ((int64_t)(r.rv ? tok : 0) * p.hq + r.hq) * 6;
  float *dg = p.dgate + r.qrow * 3;
  float sig[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) sig[c] = r.rv ? sigmoidf_(p.gates[r.qrow * 3 + c]) : 0.f;

  // compression: compressed keys b with (b + 1) 64 <= t + 1
  {
    const int nc = (wt_last + 1) / kBlk;
    const int n_tiles = (nc + kBlk - 1) / kBlk;
    auto walk = [&](auto pass, auto f) {
      lockstep<D, decltype(pass)::value>(
          n_tiles, [&](int i) { return p.tile_c + ((int64_t)g * p.n_ctile + i) * E; }, lds0, lds1,
          [&](int i, const uint16_t *b) {
            const int b0 = i * kBlk + 4 * grp;
            f(b, b + SEC, [&](int kt, int e) { return (b0 + 16 * kt + e + 1) * kBlk <= tok + 1; });
          },
          wv, lane);
    };
    q_branch<D>(p, walk, qf, of, dqa, r.rv, r.qrow, sig[0], sl2, stat, dg, lane);
  }
  bool ring_bad = false;  // a bounded wait of the selection ring gave up
  // selection: the union of the workgroup's lists, each wave computing the
  // tiles its tokens chose (rows masked to their own token's blocks, keys
  // j <= t)
  {
    int lst[TP];
#pragma unroll
    for (int q = 0; q < TP; ++q) {
      const int tq = t_first + q;
      int b = kSentinel;
      if (tq <= t_last && lane < p.topk) {
        const int32_t e = p.sel[((int64_t)tq * p.hkv + g) * p.topk + lane];
        b = sel_entry_valid(e, tq) ? (int)e : kSentinel;
      }
      lst[q] = b;
    }
    const int n_words = (p.n_vtile + 31) / 32;
    for (int w = tid; w < n_words; w += 64 * kQWaves) ubits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TP; ++q)
      if (lst[q] != kSentinel) atomicOr(&ubits[lst[q] >> 5], 1u << (lst[q] & 31));
    __syncthreads();
    if (wv == 0) {  // compact the bitmask into the ascending union
      int base = 0;
      for (int w0 = 0; w0 < n_words; w0 += 64) {
        uint32_t bits = w0 + lane < n_words ? ubits[w0 + lane] : 0u;
        const int c = __popc(bits);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(incl, o);
          if (lane >= o) incl += v;
        }
        int at = base + incl - c;
        if (w0 + lane < n_words) wpre[w0 + lane] = (int16_t)at;
        while (bits) {
          ulist[at++] = (uint16_t)(32 * (w0 + lane) + __ffs(bits) - 1);
          bits &= bits - 1u;
        }
        base += __shfl(incl, 63);
      }
      if (lane == 0) n_union = base;
    }
    __syncthreads();
    const int nu = n_union, tau = r.tau;
    // Ring walk: the union's tiles pass through three LDS slots and each wave
    // walks only the positions its tokens chose, at its own pace (no
    // workgroup barrier per tile). A wave that would wait copies instead: it
    // claims the next union tile whose slot every wave has left (compare-and-
    // swap on rnext), copies it, waits for its own copies and publishes it in
    // the slot's ready word (rready[s] = position + 1); rpass[w] = first
    // position wave w may still read. Waits are bounded: a wave that gives up
    // flags the status word and writes NaN gradients.
    constexpr int RS = 3;
    const uint16_t *tv = p.tile_v + (int64_t)g * p.n_vtile * E;
    auto slot_of = [&](int j) -> uint16_t * { const int sl = j % RS; return sl == 0 ? lds0 : sl == 1 ? lds1 : lds2; };
    auto try_copy = [&]() -> bool {
      const int j = __builtin_amdgcn_readfirstlane(lds_load(&rnext));
      if (j >= nu) return false;
      const int pv = lane < kQWaves ? lds_load(&rpass[lane]) : 0x7fffffff;
      int mn = pv;
#pragma unroll
      for (int q = 0; q < kQWaves; ++q) mn = min(mn, __builtin_amdgcn_readlane(pv, q));
      if (j > mn + RS - 1) return false;
      int won = 0;
      if (lane == 0) won = atomicCAS(&rnext, j, j + 1) == j;
      if (!__builtin_amdgcn_readfirstlane(won)) return false;
      const int blk = __builtin_amdgcn_readfirstlane((int)ulist[j]);
      asm volatile("" ::: "memory");
      dma_pieces<E / 512>(tv + (int64_t)blk * E, slot_of(j), lane);
      wait_vm_c<0>();
      asm volatile("" ::: "memory");
      if (lane == 0) lds_store(&rready[j % RS], j + 1);
      return true;
    };
    auto walk = [&](auto pass, auto f) {
      __syncthreads();  // every wave has left the slots of the previous walk
      if (tid < kQWaves) rpass[tid] = 0;
      if (tid < RS) rready[tid] = 0;
      if (tid == 0) rnext = 0;
      __syncthreads();
      int cur[TP], nxt[TP], last = -1;
#pragma unroll
      for (int q = 0; q < TP; ++q) {
        cur[q] = 0;
        nxt[q] = __builtin_amdgcn_readlane(lst[q], 0);
      }
      for (;;) {
        int u = kSentinel;
#pragma unroll
        for (int q = 0; q < TP; ++q) u = min(u, nxt[q]);
        if (u == kSentinel) break;
        uint32_t need = 0u;
#pragma unroll
        for (int q = 0; q < TP; ++q) {
          if (nxt[q] == u) {
            need |= 1u << q;
            ++cur[q];
            nxt[q] = cur[q] < p.topk ? __builtin_amdgcn_readlane(lst[q], cur[q]) : kSentinel;
          }
        }
        const uint32_t wbits = ubits[u >> 5];
        const int pos = __builtin_amdgcn_readfirstlane((int)wpre[u >> 5] + __popc(wbits & ((1u << (u & 31)) - 1u)));
        if (pos <= last) continue;  // a list out of ascending order: its slot may be gone
        last = pos;
        if (lane == 0) lds_store(&rpass[wv], pos);
        for (int spins = 0; lds_load(&rready[pos % RS]) != pos + 1;) {
          if (!try_copy()) __builtin_amdgcn_s_sleep(1);
          if (++spins > p.spin_limit) { ring_bad = true; break; }
        }
        asm volatile("" ::: "memory");
        const uint16_t *b = slot_of(pos);
        const bool rowneed = r.rv && ((need >> tau) & 1u);
        const int j0 = u * kBlk + 4 * grp;
        f(b, b + SEC, [&](int kt, int e) { return rowneed && j0 + 16 * kt + e <= tok; });
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's slot reads have returned
      if (lane == 0) lds_store(&rpass[wv], nu);
      for (int spins = 0; __builtin_amdgcn_readfirstlane(lds_load(&rnext)) < nu;) {  // copy for the rest
        if (!try_copy()) __builtin_amdgcn_s_sleep(1);
        if (++spins > p.spin_limit) { ring_bad = true; break; }
      }
    };
    q_branch<D>(p, walk, qf, of, dqa, r.rv, r.qrow, sig[1], sl2, stat + 2, dg + 1, lane);
    __syncthreads();  // no wave still reads a ring slot when the next branch copies into lds0 / lds1
  }
  // sliding window: keys t - w < j <= t
  {
    const int lo = max(0, wt_first - p.window + 1) / kBlk, hi = wt_last / kBlk;
    const int w = p.window;
    auto walk = [&](auto pass, auto f) {
      lockstep<D, decltype(pass)::value>(
          hi - lo + 1, [&](int i) { return p.tile_v + ((int64_t)g * p.n_vtile + lo + i) * E; }, lds0, lds1,
          [&](int i, const uint16_t *b) {
            const int j0 = (lo + i) * kBlk + 4 * grp;
            f(b, b + SEC, [&](int kt, int e) {
              const int j = j0 + 16 * kt + e;
              return j <= tok && j > tok - w;
            });
          },
          wv, lane);
    };
    q_branch<D>(p, walk, qf, of, dqa, r.rv, r.qrow, sig[2], sl2, stat + 4, dg + 2, lane);
  }
  if (ring_bad && lane == 0 && p.status) atomicOr(p.status, kStatusWaitGaveUp);
  const float dqs = ring_bad ? __builtin_nanf("") : p.scale;
  if (r.rv) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4 *>(p.dq + r.qrow * D + 16 * dt + 4 * grp) = dqa[dt] * dqs;
  }
}

// Text rows: dense causal attention over every earlier position, split
// over the key tiles so that the few text rows still fill the chip. A
// workgroup is (split, group, kQWaves tiles of 16/G text tokens) and walks
// its split's share of the position tiles in lockstep. Pass 1 writes the
// split's (max, sum, unnormalised o) per row; bwd_qtmerge combines the
// splits into the row statistics; pass 2 writes the split's share of dq,
// which bwd_qtsum adds in split order.
template <int D, int G>
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(2))) void bwd_qt_kernel(BwdParams p,
                                                                                                     int n_qt,
                                                                                                     int pass) {
  using R = QRows<D, G, true>;
  constexpr int TP = R::TP, DT = D / 16, SEC = BwdTile<D>::SEC, E = BwdTile<D>::E, TW = TP * kQWaves;
  __shared__ __attribute__((aligned(16))) uint16_t lds0[2 * SEC], lds1[2 * SEC];  // the two step buffers
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_grp = (n_qt + kQWaves - 1) / kQWaves;
  const int wg = blockIdx.x;
  const int qg = wg % n_grp, g = (wg / n_grp) % p.hkv, sp = wg / (n_grp * p.hkv);
  const int qt = qg * kQWaves + wv;
  const R r(p, qt, g, lane);
  const int n_text = (int)(p.n - p.n_vis);
  const int wt_last = min(qg * TW + TW, n_text) - 1;
  const int64_t pos_last = wt_last < p.v0 ? (int64_t)wt_last : (int64_t)wt_last + p.n_vis;
  const int n_tiles = (int)(pos_last / kBlk) + 1;
  const int lo = (int)((int64_t)sp * n_tiles / p.n_tsplit), hi = (int)((int64_t)(sp + 1) * n_tiles / p.n_tsplit);
  const float sl2 = p.scale * kLog2e;
  const int grp = r.grp;
  const int64_t mypos = r.pos;
  const int64_t trow = (int64_t)(r.rv ? r.tok : 0) * p.hq + r.hq;  // text row x head
  u16x8 qf[D / 32], of[D / 32];
  q_operands<D>(p, r.rv, r.qrow, qf, of, lane);
  auto tile_of = [&](int i) { return p.tile_p + ((int64_t)g * p.n_ptile + lo + i) * E; };
  if (pass == 1) {
    f32x4 oa[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oa[dt] = zero4();
    float m = -INFINITY, l = 0.f;
    lockstep<D, 1>(hi - lo, tile_of, lds0, lds1, [&](int i, const uint16_t *b) {
      const int64_t k0 = (int64_t)(lo + i) * kBlk + 4 * grp;
      q_pass1<D>(b, b + SEC, qf, oa, m, l, sl2, [&](int kt, int e) { return k0 + 16 * kt + e <= mypos; }, lane);
    }, wv, lane);
    const float L = grp_sum(l);
    if (r.rv) {
      float *part = p.tpart + ((int64_t)sp * n_text * p.hq + trow) * (D + 2);
      if (grp == 0) {
        part[0] = m;
        part[1] = L;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[2 + 16 * dt + 4 * grp + i] = oa[dt][i];
      }
    }
  } else {
    const float lse2 = r.rv ? p.tstat[trow * 2] : -INFINITY, dd = r.rv ? p.tstat[trow * 2 + 1] : 0.f;
    f32x4 dqa[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqa[dt] = zero4();
    lockstep<D, 2>(hi - lo, tile_of, lds0, lds1, [&](int i, const uint16_t *b) {
      const int64_t k0 = (int64_t)(lo + i) * kBlk + 4 * grp;
      q_pass2<D>(b, b + SEC, qf, of, dqa, lse2, dd, 1.f, sl2,
                 [&](int kt, int e) { return k0 + 16 * kt + e <= mypos; }, lane);
    }, wv, lane);
    if (r.rv) {
      float *dst = p.tpart + ((int64_t)sp * n_text * p.hq + trow) * D;  // pass-1 partials are merged by now
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt + 4 * grp) = dqa[dt];
    }
  }
}

// One workgroup of D threads per (text row, head): the splits' partials
// combined into the row's log2-sum-exp and dout . o; text rows get no gate
// gradient.
template <int D>
__global__ __launch_bounds__(D) void bwd_qtmerge_kernel(BwdParams p) {
  __shared__ float red[D / 64];
  const int64_t trow = blockIdx.x;  // text token x Hq + head
  const int d = threadIdx.x, n_text = (int)(p.n - p.n_vis);
  const int64_t stride = (int64_t)n_text * p.hq * (D + 2);
  const float *part = p.tpart + trow * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < p.n_tsplit; ++s) M = fmaxf(M, part[s * stride]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < p.n_tsplit; ++s) {
    const float ms = part[s * stride];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    L += part[s * stride + 1] * w;
    o += part[s * stride + 2 + d] * w;
  }
  const int64_t tok = trow / p.hq, h = trow % p.hq;
  const int64_t pos = tok < p.v0 ? tok : tok + p.n_vis;
  float x = L > 0.f ? h16_to_f32(f2h_bits(p.dout[(pos * p.hq + h) * D + d])) * o / L : 0.f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if ((d & 63) == 0) red[d >> 6] = x;
  __syncthreads();
  if (d == 0) {
    float dd = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) dd += red[w];
    p.tstat[trow * 2] = L > 0.f ? M + __log2f(L) : -INFINITY;
    p.tstat[trow * 2 + 1] = dd;
  }
  if (d < 3) p.dgate[(pos * p.hq + h) * 3 + d] = 0.f;
}

// dq of the text rows: the splits' shares added in split order.
template <int D>
__global__ __launch_bounds__(D) void bwd_qtsum_kernel(BwdParams p) {
  const int64_t trow = blockIdx.x;
  const int d = threadIdx.x, n_text = (int)(p.n - p.n_vis);
  const int64_t stride = (int64_t)n_text * p.hq * D;
  float acc = 0.f;
  for (int s = 0; s < p.n_tsplit; ++s) acc += p.tpart[s * stride + trow * D + d];
  const int64_t tok = trow / p.hq, h = trow % p.hq;
  const int64_t pos = tok < p.v0 ? tok : tok + p.n_vis;
  p.dq[(pos * p.hq + h) * D + d] = acc * p.scale;
}

// -------------------------------------------------------------- key side
// Query tokens walked by a key-side workgroup: tokens a + i (range) or
// list[i], i < n; `mask` picks the visibility rule, `br` the branch whose
// statistics and gate apply.
enum { kMaskWin = 0, kMaskSel = 1, kMaskAll = 2, kMaskTxt = 3, kMaskCmp = 4 };
struct TokSrc {
  int a, n;
  const int32_t *list;
  int mask, br;  // br: 0..2 vision branch, 3 text rows
};

// Rows of one step (32 at most: TS tokens x G heads), staged row-major in
// LDS by the whole workgroup (fp16 copies of q and dout) with each row's
// statistics. The rows are the A operands of S = Q K^T and dP = dO V^T as
// stored, and of dV^T = dO^T P and dK^T = Q^T dS through the gfx950
// transposing LDS read (ds_read_b64_tr_b16), so no transposed copy is
// staged. Row stride D + 24 elements: both the 16-byte row reads and the
// transposing reads of 16 lanes fall in distinct banks.
template <int D>
struct KvStage {
  static constexpr int RS = D + 24;
  uint16_t qs[32][RS], ds_[32][RS];
  float l2[32], dd[32], sig[32];
  int tok[32];
};

// A operand (16 dims x 32 rows) of a product over the step's rows from a
// row-major staged array: lane l takes dim 16 dt + (l % 16) and, as its
// eight k-slots, rows 4 (l / 16) + j and 16 + 4 (l / 16) + j (j < 4) -- the
// row order of the P / dS B operand. Each transposing read hands lane i of a
// 16-lane group element (i % 4) of the 8 bytes that lane (i / 4 + 4 j)
// addressed, so lane s addresses row 4 g + s / 4, dims 16 dt + 4 (s % 4).
template <int D>
__device__ __forceinline__ u16x8 kv_tr_frag(const uint16_t (*arr)[KvStage<D>::RS], int dt, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const uint16_t *p0 = &arr[4 * g + (s >> 2)][16 * dt + 4 * (s & 3)];
  const uint16_t *p1 = &arr[16 + 4 * g + (s >> 2)][16 * dt + 4 * (s & 3)];
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p1);
  return u16x8{(uint16_t)a[0], (uint16_t)a[1], (uint16_t)a[2], (uint16_t)a[3],
               (uint16_t)b[0], (uint16_t)b[1], (uint16_t)b[2], (uint16_t)b[3]};
}

// One thread's share of a step's rows: row r = tid / 8 (token r / G of the
// step, head r % G), dims seg PER .. +PER-1 with seg = tid % 8, loaded from
// global memory one step ahead and stored into the other LDS buffer after
// the current step's products.
template <int D>
struct KvRowRegs {
  static constexpr int PER = D / 8;
  u16x8 q[PER / 8];
  f32x4 d[PER / 4];
  float l2, dd, sg;
  int tok;
};

// The query token of this thread's row in step `step` (-1: no row).
template <int G>
__device__ __forceinline__ int kv_tok(const TokSrc &src, int step, int tid) {
  constexpr int TS = 32 / G;
  const int r = tid >> 3, tau = r / G, i = step * TS + tau;
  if (r >= TS * G || i >= src.n) return -1;
  return src.list ? src.list[i] : src.a + i;
}

template <int D, int G>
__device__ __forceinline__ void kv_load(const BwdParams &p, const TokSrc &src, int tok, int g, int tid,
                                        KvRowRegs<D> &rr) {
  constexpr int PER = D / 8;  // dims per thread
  const int r = tid >> 3, seg = tid & 7;
  const int hh = r % G;
  const bool ok = tok >= 0;
  int64_t qrow = 0;
  if (ok) {
    const int64_t pos = src.br == 3 ? (tok < p.v0 ? (int64_t)tok : (int64_t)tok + p.n_vis) : p.v0 + tok;
    qrow = pos * p.hq + g * G + hh;
  }
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) rr.q[c] = ok ? *reinterpret_cast<const u16x8 *>(p.q + qrow * D + seg * PER + 8 * c)
                                                 : zero8();
#pragma unroll
  for (int c = 0; c < PER / 4; ++c)
    rr.d[c] = ok ? *reinterpret_cast<const f32x4 *>(p.dout + qrow * D + seg * PER + 4 * c) : zero4();
  rr.tok = tok;
  rr.l2 = INFINITY;
  rr.dd = 0.f;
  rr.sg = 0.f;
  if (ok && seg == 0) {
    const int hq = g * G + hh;
    if (src.br == 3) {
      const float *st = p.tstat + ((int64_t)tok * p.hq + hq) * 2;
      rr.l2 = st[0];
      rr.dd = st[1];
      rr.sg = 1.f;
    } else {
      const float *st = p.vstat + ((int64_t)tok * p.hq + hq) * 6 + 2 * src.br;
      rr.l2 = st[0];
      rr.dd = st[1];
      rr.sg = sigmoidf_(p.gates[qrow * 3 + src.br]);
    }
  }
}

template <int D>
__device__ __forceinline__ void kv_store(KvStage<D> &sm, const KvRowRegs<D> &rr, int tid, int32_t *status) {
  constexpr int PER = D / 8;
  const int r = tid >> 3, seg = tid & 7;
  bool bad = false;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const u16x8 q8 = bf2h8(rr.q[c]);
    const u16x8 d8 = pack_p(rr.d[2 * c], rr.d[2 * c + 1]);
    bad |= any_nonfinite8(q8) || any_nonfinite8(d8);
    *reinterpret_cast<u16x8 *>(&sm.qs[r][seg * PER + 8 * c]) = q8;
    *reinterpret_cast<u16x8 *>(&sm.ds_[r][seg * PER + 8 * c]) = d8;
  }
  if (bad) atomicOr(status, kStatusRange);
  if (seg == 0) {
    float l2 = rr.l2, sg = rr.sg;
    if (l2 == -INFINITY) {  // the row has no keys in this branch
      l2 = INFINITY;
      sg = 0.f;
    }
    sm.l2[r] = l2;
    sm.dd[r] = rr.dd;
    sm.sig[r] = sg;
    sm.tok[r] = rr.tok;
  }
}

// One step for one wave (16 keys of the tile): kf / vf hold the keys' K and
// V rows as B operands; key is this lane's key index in the mask's space.
template <int D>
__device__ __forceinline__ void kv_step(const KvStage<D> &sm, const u16x8 (&kf)[D / 32], const u16x8 (&vf)[D / 32],
                                        f32x4 (&dkt)[D / 16], f32x4 (&dvt)[D / 16], int key, int mask, int window,
                                        float sl2, int lane) {
  const int r16 = lane & 15, grp = lane >> 4;
  f32x4 s[2], dp[2];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    s[rs] = zero4();
    dp[rs] = zero4();
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const u16x8 qa = *reinterpret_cast<const u16x8 *>(&sm.qs[16 * rs + r16][32 * ds + 8 * grp]);
      const u16x8 da = *reinterpret_cast<const u16x8 *>(&sm.ds_[16 * rs + r16][32 * ds + 8 * grp]);
      s[rs] = mfma_f16(qa, kf[ds], s[rs]);
      dp[rs] = mfma_f16(da, vf[ds], dp[rs]);
    }
  }
  f32x4 pm[2], dsm[2];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rs + 4 * grp + i;
      const int t = sm.tok[row];
      bool ok;
      switch (mask) {
        case kMaskWin: ok = t >= 0 && key <= t && key > t - window; break;
        case kMaskSel: ok = t >= 0 && key <= t; break;
        case kMaskAll: ok = t >= 0; break;
        case kMaskTxt: ok = t >= 0 && key <= t; break;
        default: ok = t >= 0 && (key + 1) * kBlk <= t + 1; break;  // compressed key
      }
      // dO of the branch is sig * dout: dV takes sig P against the staged dout
      const float pv = ok ? sm.sig[row] * __builtin_amdgcn_exp2f(fmaf(s[rs][i], sl2, -sm.l2[row])) : 0.f;
      pm[rs][i] = pv;
      dsm[rs][i] = pv * (dp[rs][i] - sm.dd[row]);
    }
  const u16x8 pp = pack_p(pm[0], pm[1]), pd = pack_p(dsm[0], dsm[1]);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const u16x8 da = kv_tr_frag<D>(sm.ds_, dt, lane);
    const u16x8 qa = kv_tr_frag<D>(sm.qs, dt, lane);
    dvt[dt] = mfma_f16(da, pp, dvt[dt]);
    dkt[dt] = mfma_f16(qa, pd, dkt[dt]);
  }
}

// Walks one token source 32 rows at a time through two LDS buffers. Loads
// run two steps ahead of the products (two register sets) and the tokens of
// the rows three steps ahead, so a row's address never waits on its list
// entry; each step's rows are stored into the free LDS buffer after the
// current step's products, one barrier a step.
template <int D, int G>
__device__ __forceinline__ void kv_walk(const BwdParams &p, KvStage<D> (&sm)[2], const TokSrc &src, int g,
                                        const u16x8 (&kf)[D / 32], const u16x8 (&vf)[D / 32], f32x4 (&dkt)[D / 16],
                                        f32x4 (&dvt)[D / 16], int key, float sl2, int tid) {
  constexpr int TS = 32 / G;
  const int n_steps = (src.n + TS - 1) / TS;
  if (n_steps == 0) return;
  KvRowRegs<D> rr[2];
  kv_load<D, G>(p, src, kv_tok<G>(src, 0, tid), g, tid, rr[0]);
  kv_load<D, G>(p, src, kv_tok<G>(src, 1, tid), g, tid, rr[1]);
  int tk_next = kv_tok<G>(src, 2, tid);
  kv_store<D>(sm[0], rr[0], tid, p.status);
  __syncthreads();
  for (int st = 0; st < n_steps; ++st) {
    if (st + 2 < n_steps) {
      if (st & 1) kv_load<D, G>(p, src, tk_next, g, tid, rr[1]);
      else kv_load<D, G>(p, src, tk_next, g, tid, rr[0]);
    }
    tk_next = kv_tok<G>(src, st + 3, tid);
    kv_step<D>(sm[st & 1], kf, vf, dkt, dvt, key, src.mask, p.window, sl2, tid & 63);
    if (st + 1 < n_steps) {
      if (st & 1) kv_store<D>(sm[0], rr[0], tid, p.status);
      else kv_store<D>(sm[1], rr[1], tid, p.status);
    }
    __syncthreads();
  }
}

// Key rows of the wave's 16 keys as B operands (lane: key l % 16, dims
// 32 ds + 8 (l / 16) .. +7), fp16.
template <int D, bool BF16>
__device__ __forceinline__ void kv_keys(const uint16_t *kb, const uint16_t *vb, int64_t row, bool valid, int hkv,
                                        int g, u16x8 (&kf)[D / 32], u16x8 (&vf)[D / 32], int lane) {
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    u16x8 a = zero8(), b = zero8();
    if (valid) {
      const int64_t o = (row * hkv + g) * D + 32 * ds + 8 * (lane >> 4);
      a = *reinterpret_cast<const u16x8 *>(kb + o);
      b = *reinterpret_cast<const u16x8 *>(vb + o);
      if constexpr (BF16) {
        a = bf2h8(a);
        b = bf2h8(b);
      }
    }
    kf[ds] = a;
    vf[ds] = b;
  }
}

// Vision blocks (workgroups 0 .. n_vtile Hkv - 1) then text tiles of 64
// text tokens: dk and dv of the tile's rows from every query that sees them.
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_kv_kernel(BwdParams p) {
  constexpr int DS = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(16))) KvStage<D> sm[2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_vwg = p.n_vtile * p.hkv;
  const bool vis = (int)blockIdx.x < n_vwg;
  const int id = vis ? (int)blockIdx.x : (int)blockIdx.x - n_vwg;
  const int tl = id / p.hkv, g = id % p.hkv;
  const int n_text = (int)(p.n - p.n_vis);
  const int key = tl * kBlk + 16 * wv + (lane & 15);  // vision index or text index
  const bool kvalid = vis ? key < p.n_vis : key < n_text;
  const int64_t krow = vis ? p.v0 + key : (key < p.v0 ? (int64_t)key : (int64_t)key + p.n_vis);
  u16x8 kf[DS], vf[DS];
  kv_keys<D, true>(p.k, p.v, krow, kvalid, p.hkv, g, kf, vf, lane);
  f32x4 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = zero4();
    dvt[dt] = zero4();
  }
  const float sl2 = p.scale * kLog2e;
  if (vis) {
    const int a = tl * kBlk;
    const int b = (int)min((int64_t)a + kBlk + p.window - 1, p.n_vis);
    kv_walk<D, G>(p, sm, TokSrc{a, b - a, nullptr, kMaskWin, 2}, g, kf, vf, dkt, dvt, key, sl2, tid);
    const int gb = g * p.n_vtile + tl;
    const int s0 = p.seloff[gb];
    kv_walk<D, G>(p, sm, TokSrc{0, p.seloff[gb + 1] - s0, p.selrows + s0, kMaskSel, 1}, g, kf, vf, dkt, dvt, key,
                  sl2, tid);
    if (n_text > p.v0)  // text rows after the vision run see every vision key
      kv_walk<D, G>(p, sm, TokSrc{(int)p.v0, n_text - (int)p.v0, nullptr, kMaskAll, 3}, g, kf, vf, dkt, dvt, key,
                    sl2, tid);
  } else {
    kv_walk<D, G>(p, sm, TokSrc{tl * kBlk, n_text - tl * kBlk, nullptr, kMaskTxt, 3}, g, kf, vf, dkt, dvt, key, sl2,
                  tid);
  }
  if (kvalid) {
    const int grp = lane >> 4;
    float *dk = p.dk + (krow * p.hkv + g) * D, *dv = p.dv + (krow * p.hkv + g) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<f32x4 *>(dk + 16 * dt + 4 * grp) = dkt[dt] * p.scale;
      *reinterpret_cast<f32x4 *>(dv + 16 * dt + 4 * grp) = dvt[dt];
    }
  }
}

// Compressed keys: workgroup (tile c, chunk, group) takes the vision tokens
// of its chunk that see any key of the tile and writes the partial
// gradients of the tile's 64 compressed keys.
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_kvc_kernel(BwdParams p) {
  constexpr int DS = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(16))) KvStage<D> sm[2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = blockIdx.x % p.hkv, chunk = (blockIdx.x / p.hkv) % p.n_chunk, c = blockIdx.x / (p.hkv * p.n_chunk);
  const int t_min = (c * kBlk + 1) * kBlk - 1;  // first token that sees the tile's first key
  const int a = max(chunk * kChunkTok, t_min), b = (int)min((int64_t)(chunk + 1) * kChunkTok, p.n_vis);
  if (a >= b) return;  // uniform: the reduction skips this chunk
  const int key = c * kBlk + 16 * wv + (lane & 15);
  const bool kvalid = key < p.n_blk;
  u16x8 kf[DS], vf[DS];
  kv_keys<D, false>(p.kc16, p.vc16, key, kvalid, p.hkv, g, kf, vf, lane);
  f32x4 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = zero4();
    dvt[dt] = zero4();
  }
  kv_walk<D, G>(p, sm, TokSrc{a, b - a, nullptr, kMaskCmp, 0}, g, kf, vf, dkt, dvt, key, p.scale * kLog2e, tid);
  const int grp = lane >> 4;
  float *dst = p.cpart + (((int64_t)c * p.n_chunk + chunk) * p.hkv + g) * 2 * kBlk * D;
  const int kr = 16 * wv + (lane & 15);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    *reinterpret_cast<f32x4 *>(dst + kr * D + 16 * dt + 4 * grp) = dkt[dt] * p.scale;
    *reinterpret_cast<f32x4 *>(dst + (kBlk + kr) * D + 16 * dt + 4 * grp) = dvt[dt];
  }
}

// dK_cmp, dV_cmp = the chunks' partial sums, added in chunk order.
template <int D>
__global__ __launch_bounds__(D) void bwd_creduce_kernel(BwdParams p) {
  const int b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv, d = threadIdx.x;
  const int c = b / kBlk, kr = b % kBlk;
  const int first = ((c * kBlk + 1) * kBlk - 1) / kChunkTok;
  float sk = 0.f, sv = 0.f;
  for (int ch = first; ch < p.n_chunk; ++ch) {
    const float *src = p.cpart + (((int64_t)c * p.n_chunk + ch) * p.hkv + g) * 2 * kBlk * D;
    sk += src[kr * D + d];
    sv += src[(kBlk + kr) * D + d];
  }
  const int64_t o = ((int64_t)b * p.hkv + g) * D + d;
  p.dkc[o] = sk;
  p.dvc[o] = sv;
}

// dW = sum over (block, group) of dK_cmp (x) mean; one workgroup of D
// threads per row i of dW (k and v maps).
template <int D>
__global__ __launch_bounds__(4 * D) void bwd_cmp_w_kernel(BwdParams p) {
  __shared__ float part[4][D];
  const int i = blockIdx.x % D, which = blockIdx.x / D, j = threadIdx.x % D, h = threadIdx.x / D;
  const float *dy = which ? p.dvc : p.dkc;
  const float *x = which ? p.vbar : p.kbar;
  // four contiguous quarters of the rows, each summed in eight interleaved
  // partial sums (sixteen rows' loads in flight), then added in quarter
  // order: a fixed order, so the result is bitwise repeatable
  const int64_t rows = (int64_t)p.n_blk * p.hkv, q = (rows + 3) / 4;
  const int64_t r0 = min(rows, h * q), r1 = min(rows, r0 + q);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  int64_t r = r0;
#pragma unroll 2
  for (; r + 8 <= r1; r += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = fmaf(dy[(r + u) * D + i], x[(r + u) * D + j], acc[u]);
  }
  for (int u = 0; r < r1; ++r, ++u) acc[u] = fmaf(dy[r * D + i], x[r * D + j], acc[u]);
  part[h][j] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (h == 0) (which ? p.dwv : p.dwk)[i * D + j] = (part[0][j] + part[1][j]) + (part[2][j] + part[3][j]);
}

// Each block's share of the tokens' gradients: W^T dK_cmp / 64 added to the
// 64 rows of dk (dv likewise); one workgroup of D threads per (block, group).
template <int D>
__global__ __launch_bounds__(D) void bwd_cmp_tok_kernel(BwdParams p) {
  __shared__ float dy[2][D];
  const int b = blockIdx.x / p.hkv, g = blockIdx.x % p.hkv, j = threadIdx.x;
  const int64_t ob = ((int64_t)b * p.hkv + g) * D;
  dy[0][j] = p.dkc[ob + j];
  dy[1][j] = p.dvc[ob + j];
  __syncthreads();
  float uk = 0.f, uv = 0.f;
  for (int i = 0; i < D; ++i) {
    uk = fmaf(bfbits2f(p.wk[i * D + j]), dy[0][i], uk);
    uv = fmaf(bfbits2f(p.wv[i * D + j]), dy[1][i], uv);
  }
  uk *= 1.f / kBlk;
  uv *= 1.f / kBlk;
  for (int r = 0; r < kBlk; ++r) {
    const int64_t o = ((p.v0 + (int64_t)b * kBlk + r) * p.hkv + g) * D + j;
    p.dk[o] += uk;
    p.dv[o] += uv;
  }
}

template <int D, int G>
hipError_t run_g(const BwdParams &p, int stage, hipStream_t st) {
  constexpr int TP = 16 / G;
  switch (stage) {
    case 7: {  // query side, vision rows
      const int n_qt = (int)((p.n_vis + TP - 1) / TP);
      const int64_t n_wg = (int64_t)((n_qt + kQWaves - 1) / kQWaves) * p.hkv;
      if (n_wg == 0) return hipSuccess;
      hipLaunchKernelGGL((bwd_q_kernel<D, G>), dim3((unsigned)((n_wg + 7) / 8 * 8)), dim3(64 * kQWaves), 0, st, p,
                         n_qt);
      break;
    }
    case 8: {  // query side, text rows: split pass 1, merge, split pass 2, sum
      const int64_t n_text = p.n - p.n_vis;
      const int n_qt = (int)((n_text + TP - 1) / TP);
      const int64_t n_wg = (int64_t)((n_qt + kQWaves - 1) / kQWaves) * p.hkv * p.n_tsplit;
      if (n_wg == 0) return hipSuccess;
      hipLaunchKernelGGL((bwd_qt_kernel<D, G>), dim3((unsigned)n_wg), dim3(64 * kQWaves), 0, st, p, n_qt, 1);
      hipLaunchKernelGGL((bwd_qtmerge_kernel<D>), dim3((unsigned)(n_text * p.hq)), dim3(D), 0, st, p);
      hipLaunchKernelGGL((bwd_qt_kernel<D, G>), dim3((unsigned)n_wg), dim3(64 * kQWaves), 0, st, p, n_qt, 2);
      hipLaunchKernelGGL((bwd_qtsum_kernel<D>), dim3((unsigned)(n_text * p.hq)), dim3(D), 0, st, p);
      break;
    }
    case 9: {  // key side: vision blocks and text tiles
      const int n_ttile = (int)((p.n - p.n_vis + kBlk - 1) / kBlk);
      const int64_t n_wg = (int64_t)(p.n_vtile + n_ttile) * p.hkv;
      if (n_wg == 0) return hipSuccess;
      hipLaunchKernelGGL((bwd_kv_kernel<D, G>), dim3((unsigned)n_wg), dim3(256), 0, st, p);
      break;
    }
    default: {  // key side: compressed keys
      const int64_t n_wg = (int64_t)p.n_ctile * p.n_chunk * p.hkv;
      if (n_wg == 0) return hipSuccess;
      hipLaunchKernelGGL((bwd_kvc_kernel<D, G>), dim3((unsigned)n_wg), dim3(256), 0, st, p);
      break;
    }
  }
  return hipGetLastError();
}

template <int D>
hipError_t run(const BwdParams &p, int stage, hipStream_t st) {
  switch (stage) {
    case 0: {  // clear the selection bitmask
      const int64_t n = (int64_t)p.hkv * p.n_vtile * p.mask_words;
      if (n > 0) hipLaunchKernelGGL(bwd_fill_kernel, dim3(1024), dim3(256), 0, st, p.selmask, n);
      break;
    }
    case 1:
      if (p.n_blk > 0) hipLaunchKernelGGL((bwd_pool_kernel<D>), dim3(p.n_blk * p.hkv), dim3(D), 0, st, p);
      break;
    case 2: {  // backward tiles
      if (p.n_vtile > 0)
        hipLaunchKernelGGL((bwd_pack_kernel<D, true>), dim3(p.n_vtile * p.hkv), dim3(256), 0, st, p.k, p.v, p.v0,
                           p.n_vis, p.hkv, p.n_vtile, p.tile_v, p.status);
      if (p.n > p.n_vis)
        hipLaunchKernelGGL((bwd_pack_kernel<D, true>), dim3(p.n_ptile * p.hkv), dim3(256), 0, st, p.k, p.v,
                           (int64_t)0, p.n, p.hkv, p.n_ptile, p.tile_p, p.status);
      if (p.n_ctile > 0)
        hipLaunchKernelGGL((bwd_pack_kernel<D, false>), dim3(p.n_ctile * p.hkv), dim3(256), 0, st, p.kc16, p.vc16,
                           (int64_t)0, (int64_t)p.n_blk, p.hkv, p.n_ctile, p.tile_c, p.status);
      break;
    }
    case 3: {  // who chose which block
      const int64_t n = p.n_vis * p.hkv * p.topk;
      if (n == 0) break;
      hipLaunchKernelGGL(bwd_selmask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
      hipLaunchKernelGGL(bwd_selcount_kernel, dim3(p.hkv * p.n_vtile), dim3(64), 0, st, p);
      hipLaunchKernelGGL(bwd_selscan_kernel, dim3(1), dim3(256), 0, st, p, p.hkv * p.n_vtile);
      hipLaunchKernelGGL(bwd_selfill_kernel, dim3(p.hkv * p.n_vtile), dim3(64), 0, st, p);
      break;
    }
    case 7: case 8: case 9: case 10:
      switch (p.hq / p.hkv) {
        case 1: return run_g<D, 1>(p, stage, st);
        case 2: return run_g<D, 2>(p, stage, st);
        case 3: return run_g<D, 3>(p, stage, st);
        case 4: return run_g<D, 4>(p, stage, st);
        case 5: return run_g<D, 5>(p, stage, st);
        case 6: return run_g<D, 6>(p, stage, st);
        case 7: return run_g<D, 7>(p, stage, st);
        case 8: return run_g<D, 8>(p, stage, st);
        default: return hipErrorInvalidValue;
      }
    case 11:
      if (p.n_blk > 0) hipLaunchKernelGGL((bwd_creduce_kernel<D>), dim3(p.n_blk * p.hkv), dim3(D), 0, st, p);
      break;
    case 12:
      hipLaunchKernelGGL((bwd_cmp_w_kernel<D>), dim3(2 * D), dim3(4 * D), 0, st, p);
      break;
    default:
      if (p.n_blk > 0) hipLaunchKernelGGL((bwd_cmp_tok_kernel<D>), dim3(p.n_blk * p.hkv), dim3(D), 0, st, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdParams &p, int d, int stage, hipStream_t st) {
  if (d == 64) return run<64>(p, stage, st);
  if (d == 128) return run<128>(p, stage, st);
  return hipErrorInvalidValue;
}

}  // namespace nsa
