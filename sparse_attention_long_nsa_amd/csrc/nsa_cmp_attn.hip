// Compression-branch attention and block importance scores.
//
// Every vision query attends to the compressed block keys/values of the
// complete blocks before it (VideoNSA paper summary page, "Method", branch
// (a); readings: a block is visible once complete, empty set -> zero output).
// The selection branch ranks blocks by an importance score taken from this
// attention (same section, branch (b)); the reading used is the sum over the
// KV group's query heads of each head's normalised probability, so the
// kernel runs two passes over the compressed keys: pass 1 finds every
// query's log-sum-exp, pass 2 forms exact probabilities, which feed the PV
// product (no running rescale needed) and, summed over the group's heads in
// registers, the frame-packed group-score rows read by the top-k kernel.
//
// Layout: one workgroup = one 64-token frame x one KV group, four waves of
// 16 tokens each; every wave carries all G query heads of its tokens, so a
// K or V^T fragment read from LDS feeds G matrix-core ops and the head sum
// of the importance score never leaves the lane. Workgroups are ordered
// heaviest (latest frame) first and interleave KV groups so that consecutive
// workgroup ids -- which land on different XCDs -- keep one group's
// compressed keys per XCD L2.
//
// Staging (bf16 inputs): the compressed keys/values are first packed into
// PackedTile chunks of 64 blocks, which stream into LDS by direct
// global->LDS copies. The two passes are two kernels: pass 1 (keys only,
// no global stores in flight) fits 256 registers, so two of its workgroups
// share a CU, each ringing keys through four chunk slots with explicit
// vmcnt waits; pass 2 (seven heads' output accumulators fill the register
// file: one wave per SIMD) writes the score rows as it goes, so it
// double-buffers and waits for all of its memory operations before each
// chunk. fp32 inputs (split operands) keep one kernel with synchronous
// staging.
#include "nsa_kernels.h"
#include "nsa_tiles.h"

namespace nsa {

namespace {

constexpr int kThreadsH = 256;  // 4 waves x 16 tokens
constexpr int kBufWord3 = 0x00020000;  // buffer resource word 3 (raw, 32-bit) on gfx9

// Folds four scaled logits (log2 units, -inf = masked) into a lane-partial
// (max, sum) pair.
__device__ __forceinline__ void fold4(float &m, float &l, const f32x4 x) {
  const float mx = fmax_nn(fmax_nn(x[0], x[1]), fmax_nn(x[2], x[3]));
  const float mn = fmax_nn(m, mx);
  if (mn == -INFINITY) return;
  l = l * exp2f(m - mn) + exp2f(x[0] - mn) + exp2f(x[1] - mn) + exp2f(x[2] - mn) + exp2f(x[3] - mn);
  m = mn;
}

// Scores of 16 compressed keys: fp16 q x fp16 keys, or (split operands, for
// fp32 inputs) bf16 q_hi*k_hi + q_hi*k_lo + q_lo*k_hi.
template <int D, int G, bool SPLIT>
__device__ __forceinline__ void scores16(f32x4 (&s)[G], const uint16_t *ks, const uint16_t *ksl, int kt,
                                         const u16x8 (&qf)[G][D / 32],
                                         const u16x8 (&ql)[SPLIT ? G : 1][D / 32], int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const u16x8 a = k_frag<D>(ks, kt, ds, lane);
    if constexpr (SPLIT) {
      const u16x8 al = k_frag<D>(ksl, kt, ds, lane);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s[h] = mfma_bf16(a, qf[h][ds], s[h]);
        s[h] = mfma_bf16(al, qf[h][ds], s[h]);
        s[h] = mfma_bf16(a, ql[h][ds], s[h]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = mfma_f16(a, qf[h][ds], s[h]);
    }
  }
}

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__(kThreadsH) void cmp_attn_kernel(CmpAttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[Tile<D>::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t ksl[SPLIT ? Tile<D>::kElems : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vt[Tile<D>::vElems];
  constexpr int DS = D / 32, DT = D / 16;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x % p.hkv;
  const int f = p.n_frames - 1 - (int)(blockIdx.x / p.hkv);
  const int t = f * kBlk + wv * 16 + row;  // this lane's query (vision-local)
  const bool tvalid = t < p.n_vis;
  const int nc_t = tvalid ? (t + 1) / kBlk : 0;  // complete blocks visible to it
  const int t_last = min(f * kBlk + kBlk - 1, p.n_vis - 1);
  const int nk = (t_last + 1) / kBlk;            // blocks any query of the frame sees
  const int64_t kvs = (int64_t)p.hkv * D;
  const uint16_t *kc = p.kc + (int64_t)g * D;
  const uint16_t *kcl = SPLIT ? p.kc_lo + (int64_t)g * D : nullptr;
  const uint16_t *vc = p.vc + (int64_t)g * D;

  u16x8 qf[G][DS];
  u16x8 ql[SPLIT ? G : 1][DS];
  {
    const int64_t q0 = (row_pos(p.vmap, p.v0, tvalid ? t : 0) * p.hq + (int64_t)g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const u16x8 raw = tvalid ? q_frag_global(p.q + q0 + h * D, ds, lane) : zero8();
        qf[h][ds] = SPLIT ? raw : bf2h8(raw);  // fp16 scores unless split
        if constexpr (SPLIT) ql[h][ds] = tvalid ? q_frag_global(p.q_lo + q0 + h * D, ds, lane) : zero8();
      }
  }

  // ---- pass 1: log-sum-exp of every (query, head)
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
  for (int c = 0; c * kBlk < nk; ++c) {
    const int nvalid = min(kBlk, nk - c * kBlk);
    __syncthreads();
    stage_k<D>(ks, kc + (int64_t)c * kBlk * kvs, kvs, nvalid, tid, kThreadsH);
    if constexpr (SPLIT) stage_k<D>(ksl, kcl + (int64_t)c * kBlk * kvs, kvs, nvalid, tid, kThreadsH);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 s[G];
      scores16<D, G, SPLIT>(s, ks, ksl, kt, qf, ql, lane);
      const int b0 = c * kBlk + 16 * kt + 4 * grp;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (b0 + i < nc_t) ? s[h][i] * p.sl2 : -INFINITY;
        fold4(m[h], l[h], x);
      }
    }
  }
  float lse2[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = grp_max(m[h]);
    const float part = (m[h] == -INFINITY) ? 0.f : l[h] * exp2f(m[h] - M);
    const float L = grp_sum(part);
    lse2[h] = (L > 0.f) ? M + log2f(L) : -INFINITY;
  }
  if (tvalid && grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) p.lse[(int64_t)t * p.hq + g * G + h] = lse2[h] * (1.0f / kLog2e);
  }

  // ---- pass 2: probabilities -> o_cmp and group scores
  f32x4 o[G][DT];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[h][dt] = zero4();
  float *gsrow = p.gs + frame_off(f, p.hkv) + (int64_t)(g * kBlk + (t - f * kBlk)) * f;
  for (int c = 0; c * kBlk < nk; ++c) {
    const int nvalid = min(kBlk, nk - c * kBlk);
    __syncthreads();
    stage_k<D>(ks, kc + (int64_t)c * kBlk * kvs, kvs, nvalid, tid, kThreadsH);
    if constexpr (SPLIT) stage_k<D>(ksl, kcl + (int64_t)c * kBlk * kvs, kvs, nvalid, tid, kThreadsH);
    stage_vt<D, false>(vt, vc + (int64_t)c * kBlk * kvs, kvs, nvalid, tid, kThreadsH);
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      f32x4 s[2][G];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kt = 2 * ks2 + kk;
        scores16<D, G, SPLIT>(s[kk], ks, ksl, kt, qf, ql, lane);
        const int b0 = c * kBlk + 16 * kt + 4 * grp;
        f32x4 gsum = zero4();
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[kk][h][i] = (b0 + i < nc_t) ? exp2f(s[kk][h][i] * p.sl2 - lse2[h]) : 0.f;
          gsum += s[kk][h];
        }
        if (tvalid) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (b0 + i < f) gsrow[b0 + i] = gsum[i];
        }
      }
      u16x8 pf[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pf[h] = pack_p(s[0][h], s[1][h]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u16x8 a = v_frag<D>(vt, dt, ks2, lane);
#pragma unroll
        for (int h = 0; h < G; ++h) o[h][dt] = mfma_f16(a, pf[h], o[h][dt]);
      }
    }
  }

  // ---- epilogue: sigmoid(g_cmp) * o_cmp as the fp16 part 0 of the row's
  // output slots (the selection kernel adds the branches and writes fp32)
  if (tvalid) {
    const int64_t r0 = row_pos(p.vmap, p.v0, t) * p.hq + (int64_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float gate = sigmoidf_(p.gates[(r0 + h) * 3 + 0]);
      float *slot = p.out + (r0 + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store_partial4<D>(slot, 0, 16 * dt + 4 * grp, o[h][dt] * gate);
    }
  }
}

// Pipelined kernels for fp16 operands (bf16 inputs); same math as above.
// The ring slots are separate LDS objects and every step names its slot at
// compile time: reads of one slot then need not wait for copies still
// landing in another.
// Both passes walk a chunk head by head as a software pipeline: the scores of
// head h+1 are issued to the matrix cores before head h's exponentials, so
// the two overlap within the one wave. The K fragments (and in pass 2 the V
// fragments) of a half chunk stay in registers across the heads. Only a
// frame's last chunk holds blocks some of its queries must not see (every
// earlier chunk ends before the frame's first block, f), so only that chunk
// runs the masked form: its score accumulators start at -inf for the hidden
// blocks (one bias per block, shared by every head) and its score rows are
// written with buffer stores whose out-of-range lanes the hardware drops.
// The other chunks start from zero accumulators and store unguarded.
template <int D, int NT, bool MASKED>
__device__ __forceinline__ void cmp_scores(const u16x8 (&kf)[NT][D / 32], const u16x8 (&q)[D / 32],
                                           const f32x4 (&bias)[NT], f32x4 (&s)[NT]) {
#pragma unroll
  for (int kt = 0; kt < NT; ++kt) s[kt] = MASKED ? bias[kt] : zero4();
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) s[kt] = mfma_f16(kf[kt][ds], q[ds], s[kt]);
}

// One chunk of pass 1, in two halves of 32 keys: a half's key fragments
// stay in registers across the heads (half a chunk keeps the kernel within
// 256 registers), with an exact running max per half and head.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void cmp_pass1_chunk(const uint16_t *ks, int c, const u16x8 (&qf)[G][D / 32],
                                                float (&m)[G], float (&l)[G], int nc_t, float sl2, int lane) {
  const int grp = lane >> 4;
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    u16x8 kf[2][D / 32];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) kf[kk][ds] = pk_k_frag<D>(ks, 2 * ks2 + kk, ds, lane);
    const int b0 = c * kBlk + 32 * ks2 + 4 * grp;  // block of element (kk, i): b0 + 16 kk + i
    f32x4 bias[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[kk][i] = (!MASKED || b0 + 16 * kk + i < nc_t) ? 0.f : -INFINITY;
    f32x4 sc[2], sn[2];
    cmp_scores<D, 2, MASKED>(kf, qf[0], bias, sc);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h + 1 < G) cmp_scores<D, 2, MASKED>(kf, qf[h + 1], bias, sn);
      float mx = sc[0][0];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmax_nn(mx, sc[kk][i]);
      // raw scores; the scale sl2 > 0 is folded into the exponent
      const float mn = fmax_nn(m[h], mx * sl2);
      const float nb = (mn == -INFINITY) ? 0.f : -mn;
      float acc = (m[h] == -INFINITY) ? 0.f : l[h] * __builtin_amdgcn_exp2f(m[h] + nb);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += __builtin_amdgcn_exp2f(fmaf(sc[kk][i], sl2, nb));
      l[h] = acc;
      m[h] = mn;
      if (h + 1 < G) {
        sc[0] = sn[0];
        sc[1] = sn[1];
      }
    }
  }
}

// gsr: buffer resource over this workgroup's score rows (64 rows of f
// floats); srow: byte offset of this lane's row. nlse2: minus each head's
// log2-sum-exp, -inf where the query sees no block.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void cmp_pass2_chunk(const uint16_t *ks, const uint16_t *vt, int c,
                                                const u16x8 (&qf)[G][D / 32], f32x4 (&o)[G][D / 16],
                                                const float (&nlse2)[G], __amdgpu_buffer_rsrc_t gsr,
                                                int srow, int f, int nc_t, float sl2, int lane) {
  const int grp = lane >> 4;
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    // keys 32*ks2 .. 32*ks2+31 of the chunk: key subtiles kt = 2*ks2 + kk
    u16x8 kf[2][D / 32], vf[D / 16];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ds = 0; ds < D / 32; ++ds) kf[kk][ds] = pk_k_frag<D>(ks, 2 * ks2 + kk, ds, lane);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = pk_v_frag<D>(vt, dt, ks2, lane);
    const int b0 = c * kBlk + 32 * ks2 + 4 * grp;  // block of element (kk, i): b0 + 16 kk + i
    f32x4 bias[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[kk][i] = (!MASKED || b0 + 16 * kk + i < nc_t) ? 0.f : -INFINITY;
    f32x4 sc[2], sn[2], gsum[2];
    cmp_scores<D, 2, MASKED>(kf, qf[0], bias, sc);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h + 1 < G) cmp_scores<D, 2, MASKED>(kf, qf[h + 1], bias, sn);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kk][i] = __builtin_amdgcn_exp2f(fmaf(sc[kk][i], sl2, nlse2[h]));
        gsum[kk] = h == 0 ? sc[kk] : gsum[kk] + sc[kk];
      }
      const u16x8 pf = pack_p(sc[0], sc[1]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[h][dt] = mfma_f16(vf[dt], pf, o[h][dt]);
      if (h + 1 < G) {
        sc[0] = sn[0];
        sc[1] = sn[1];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = b0 + 16 * kk + i;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gsum[kk][i]), gsr,
                                              (!MASKED || b < f) ? srow + 4 * b : 0x7ffffff0, 0, 0);
      }
  }
}

// Pass 1 for fp16 operands: every query's log-sum-exp over the compressed
// keys, written to lse in log2 units (pass 2 reads it there and leaves it in
// natural-log units). It is a kernel of its own so that it fits 256
// registers (the query fragments, one chunk's key fragments, two heads'
// scores): two workgroups share a CU, and one wave's exponentials run while
// the other's products are on the matrix cores. Keys ring through four slots
// (three chunks in flight) with explicit vmcnt waits; no other memory
// operation is in flight during the walk.
template <int D, int G>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2))) void cmp_lse_kernel(
    CmpAttnParams p) {
  using T = PackedTile<D>;
  constexpr int KE = T::KE, SE = T::KE + T::VE;
  constexpr int PK = KE / 512 / 4;  // pieces per wave of a key tile
  __shared__ __attribute__((aligned(16))) uint16_t r0[KE], r1[KE], r2[KE], r3[KE];
  constexpr int DS = D / 32;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x % p.hkv;
  const int f = p.n_frames - 1 - (int)(blockIdx.x / p.hkv);
  const int t = f * kBlk + wv * 16 + row;  // this lane's query (vision-local)
  const bool tvalid = t < p.n_vis;
  const int nc_t = tvalid ? (t + 1) / kBlk : 0;  // complete blocks visible to it
  const int t_last = min(f * kBlk + kBlk - 1, p.n_vis - 1);
  const int nk = (t_last + 1) / kBlk;            // blocks any query of the frame sees
  const int nch = (nk + kBlk - 1) / kBlk;        // packed chunks holding them
  const int off = __builtin_amdgcn_readfirstlane(wv * PK * 512);  // wave-uniform, scalar
  const uint16_t *cg = p.kvc + (int64_t)g * p.n_cch * SE + off;

  u16x8 qf[G][DS];
  {
    const int64_t q0 = (row_pos(p.vmap, p.v0, tvalid ? t : 0) * p.hq + (int64_t)g * G) * D;
    bool ovf = false;  // a query past fp16's range (flagged in the status word)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        qf[h][ds] = tvalid ? bf2h8(q_frag_global(p.q + q0 + h * D, ds, lane)) : zero8();
#pragma unroll
        for (int e = 0; e < 8; ++e) ovf |= h16_nonfinite(qf[h][ds][e]);
      }
    if (ovf && p.status) atomicOr(p.status, kStatusRange);
  }

  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
  // Every step issues exactly PK copies, so "chunk c landed" is always
  // vmcnt <= 2 * PK. Past the last chunk the copies repeat chunk 0 into
  // slots that are never read again.
#define NSA_ISSUE_K_OR_PAD(DST, C) dma_pieces<PK>(cg + (int64_t)((C) < nch ? (C) : 0) * SE, (DST) + off, lane)
#define NSA_P1_STEP(CUR, NXT)                                             \
  {                                                                       \
    wait_vm_c<2 * PK>();                                                  \
    bare_barrier();                                                       \
    NSA_ISSUE_K_OR_PAD(NXT, c + 3);                                       \
    cmp_pass1_chunk<D, G, false>(CUR, c, qf, m, l, nc_t, p.sl2, lane);    \
    if (++c >= nch - 1) break;                                            \
  }
  if (nch > 0) {
    NSA_ISSUE_K_OR_PAD(r0, 0);
    NSA_ISSUE_K_OR_PAD(r1, 1);
    NSA_ISSUE_K_OR_PAD(r2, 2);
  }
  for (int c = 0; c < nch - 1;) {  // every chunk but the last: nothing hidden
    NSA_P1_STEP(r0, r3)
    NSA_P1_STEP(r1, r0)
    NSA_P1_STEP(r2, r1)
    NSA_P1_STEP(r3, r2)
  }
#undef NSA_P1_STEP
#undef NSA_ISSUE_K_OR_PAD
  wait_vm_c<0>();  // the last chunk and every padding copy have landed
  if (nch > 0) {
    bare_barrier();
    const int cl = nch - 1, sl = cl & 3;
    const uint16_t *ks = sl == 0 ? r0 : sl == 1 ? r1 : sl == 2 ? r2 : r3;
    cmp_pass1_chunk<D, G, true>(ks, cl, qf, m, l, nc_t, p.sl2, lane);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = grp_max(m[h]);
    const float part = (m[h] == -INFINITY) ? 0.f : l[h] * exp2f(m[h] - M);
    const float L = grp_sum(part);
    m[h] = (L > 0.f) ? M + log2f(L) : -INFINITY;
  }
  if (tvalid && grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) p.lse[(int64_t)t * p.hq + g * G + h] = m[h];
  }
}

// Pass 2 for fp16 operands: probabilities from pass 1's log-sum-exp ->
// o_cmp and the group scores. The score rows are stored as the loop goes,
// so each chunk waits for all of this wave's memory operations (double
// buffering: chunk c+1 flies during chunk c).
template <int D, int G>
__global__ __launch_bounds__(kThreadsH) void cmp_attn_dma_kernel(CmpAttnParams p) {
  using T = PackedTile<D>;
  constexpr int KE = T::KE, SE = T::KE + T::VE;
  constexpr int PK = KE / 512 / 4;  // pieces per wave of a key tile (a value tile alike)
  static_assert(T::VE == KE, "square tiles");
  // two chunk slots of (K, V^T), double-buffered
  __shared__ __attribute__((aligned(16))) uint16_t r0[KE], r1[KE], r2[KE], r3[KE];
  constexpr int DS = D / 32, DT = D / 16;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int g = blockIdx.x % p.hkv;
  const int f = p.n_frames - 1 - (int)(blockIdx.x / p.hkv);
  const int t = f * kBlk + wv * 16 + row;  // this lane's query (vision-local)
  const bool tvalid = t < p.n_vis;
  const int nc_t = tvalid ? (t + 1) / kBlk : 0;  // complete blocks visible to it
  const int t_last = min(f * kBlk + kBlk - 1, p.n_vis - 1);
  const int nk = (t_last + 1) / kBlk;            // blocks any query of the frame sees
  const int nch = (nk + kBlk - 1) / kBlk;        // packed chunks holding them
  const int off = __builtin_amdgcn_readfirstlane(wv * PK * 512);  // wave-uniform, scalar
  const uint16_t *cg = p.kvc + (int64_t)g * p.n_cch * SE + off;

  u16x8 qf[G][DS];
  float lse2[G];  // log2 units, from pass 1
  {
    const int64_t q0 = (row_pos(p.vmap, p.v0, tvalid ? t : 0) * p.hq + (int64_t)g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qf[h][ds] = tvalid ? bf2h8(q_frag_global(p.q + q0 + h * D, ds, lane)) : zero8();
    const float *lr = p.lse + (int64_t)(tvalid ? t : 0) * p.hq + g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) lse2[h] = tvalid ? lr[h] : -INFINITY;
  }

  f32x4 o[G][DT];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[h][dt] = zero4();
  // the workgroup's score rows: 64 rows (padding rows of a partial frame
  // included) of f floats; stores past a row's end fall outside and are dropped
  const __amdgpu_buffer_rsrc_t gsr = __builtin_amdgcn_make_buffer_rsrc(
      p.gs + frame_off(f, p.hkv) + (int64_t)g * kBlk * f, 0, kBlk * f * (int)sizeof(float), kBufWord3);
  const int srow = (t - f * kBlk) * f * (int)sizeof(float);
  float nlse2[G];  // -lse2; -inf where no block is visible (every probability 0)
#pragma unroll
  for (int h = 0; h < G; ++h) nlse2[h] = (lse2[h] == -INFINITY) ? -INFINITY : -lse2[h];
#define NSA_ISSUE_KV(DK, DV, C)                                           \
  {                                                                       \
    dma_pieces<PK>(cg + (int64_t)(C) * SE, (DK) + off, lane);             \
    dma_pieces<PK>(cg + (int64_t)(C) * SE + KE, (DV) + off, lane);        \
  }
  if (nch > 0) NSA_ISSUE_KV(r0, r1, 0);
#define NSA_P2_STEP(CK, CV, NK, NV)                                       \
  {                                                                       \
    wait_vm_c<0>();                                                       \
    bare_barrier();                                                       \
    NSA_ISSUE_KV(NK, NV, c + 1);                                          \
    cmp_pass2_chunk<D, G, false>(CK, CV, c, qf, o, nlse2, gsr, srow, f, nc_t, p.sl2, lane); \
    if (++c >= nch - 1) break;                                            \
  }
  for (int c = 0; c < nch - 1;) {  // every chunk but the last: nothing hidden
    NSA_P2_STEP(r0, r1, r2, r3)
    NSA_P2_STEP(r2, r3, r0, r1)
  }
#undef NSA_P2_STEP
#undef NSA_ISSUE_KV
  if (nch > 0) {  // the last chunk, in slot pair (nch - 1) mod 2
    wait_vm_c<0>();
    bare_barrier();
    const int cl = nch - 1;
    const uint16_t *ck = (cl & 1) ? r2 : r0, *cv = (cl & 1) ? r3 : r1;
    cmp_pass2_chunk<D, G, true>(ck, cv, cl, qf, o, nlse2, gsr, srow, f, nc_t, p.sl2, lane);
  }

  // ---- epilogue: sigmoid(g_cmp) * o_cmp as the fp16 part 0 of the row's
  // output slots (the selection kernel adds the branches and writes fp32);
  // the log-sum-exp leaves in natural-log units (every lane of the row has
  // read it: the loads returned before the walk used them)
  if (tvalid) {
    const int64_t r0w = row_pos(p.vmap, p.v0, t) * p.hq + (int64_t)g * G;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float gate = sigmoidf_(p.gates[(r0w + h) * 3 + 0]);
      float *slot = p.out + (r0w + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store_partial4<D>(slot, 0, 16 * dt + 4 * grp, o[h][dt] * gate);
    }
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) p.lse[(int64_t)t * p.hq + g * G + h] = lse2[h] * (1.0f / kLog2e);
    }
  }
}

template <int D, int G, bool SPLIT>
hipError_t run(const CmpAttnParams &p, hipStream_t st) {
  const unsigned nwg = (unsigned)p.n_frames * (unsigned)p.hkv;
  if (nwg == 0) return hipSuccess;
  if constexpr (SPLIT) {
    hipLaunchKernelGGL((cmp_attn_kernel<D, G, true>), dim3(nwg), dim3(kThreadsH), 0, st, p);
  } else {
    if (!p.kvc && p.n_cch > 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cmp_lse_kernel<D, G>), dim3(nwg), dim3(kThreadsH), 0, st, p);
    hipLaunchKernelGGL((cmp_attn_dma_kernel<D, G>), dim3(nwg), dim3(kThreadsH), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cmp_attn(const CmpAttnParams &p, int d, int G, bool split, hipStream_t st) {
  if (split) {
    if (d == 64) {
      switch (G) {
        case 1: return run<64, 1, true>(p, st);
        case 2: return run<64, 2, true>(p, st);
        case 3: return run<64, 3, true>(p, st);
        case 4: return run<64, 4, true>(p, st);
        case 5: return run<64, 5, true>(p, st);
        case 6: return run<64, 6, true>(p, st);
        case 7: return run<64, 7, true>(p, st);
        case 8: return run<64, 8, true>(p, st);
      }
    } else {
      switch (G) {
        case 1: return run<128, 1, true>(p, st);
        case 2: return run<128, 2, true>(p, st);
        case 3: return run<128, 3, true>(p, st);
        case 4: return run<128, 4, true>(p, st);
      }
    }
    return hipErrorInvalidValue;
  }
  if (d == 64) {
    switch (G) {
      case 1: return run<64, 1, false>(p, st);
      case 2: return run<64, 2, false>(p, st);
      case 3: return run<64, 3, false>(p, st);
      case 4: return run<64, 4, false>(p, st);
      case 5: return run<64, 5, false>(p, st);
      case 6: return run<64, 6, false>(p, st);
      case 7: return run<64, 7, false>(p, st);
      case 8: return run<64, 8, false>(p, st);
    }
  } else {
    switch (G) {
      case 1: return run<128, 1, false>(p, st);
      case 2: return run<128, 2, false>(p, st);
      case 3: return run<128, 3, false>(p, st);
      case 4: return run<128, 4, false>(p, st);
      case 5: return run<128, 5, false>(p, st);
      case 6: return run<128, 6, false>(p, st);
      case 7: return run<128, 7, false>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

bool supported_heads(int d, int G, bool split) {
  if (d != 64 && d != 128) return false;
  if (G < 1 || G > 8) return false;
  if (d == 128 && G > 7) return false;     // G x 16 x 128 accumulators per wave
  if (split && G * d > 512) return false;  // split operands double the query registers
  return true;
}

}  // namespace nsa
