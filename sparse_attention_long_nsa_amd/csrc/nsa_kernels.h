// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include "nsa_common.h"

namespace nsa {

// Offset (in floats) of frame f's block in the frame-packed group-score
// buffer: frame f's 64 tokens x Hkv groups each own a row of f scores, one
// per candidate block 0 .. f-1 (the frame's own block is never a candidate).
__host__ __device__ __forceinline__ int64_t frame_off(int64_t f, int hkv) {
  return (int64_t)kBlk * hkv * (f * (f - 1) / 2);
}

// Global position of row i of a token set (the vision tokens, or the text
// tokens): map[i] when the set is scattered over several runs of the
// sequence, else row0 + i.
__device__ __forceinline__ int64_t row_pos(const int32_t *map, int64_t row0, int64_t i) {
  return map ? (int64_t)map[i] : row0 + i;
}

struct PoolJob {
  const void *x;     // first row of the pooled run, [n_rows, n_heads, d]
  const void *w;     // [d, d]
  int n_heads;
  int64_t n_blk;
  uint16_t *out_hi;  // bf16 rounding of the result (or null)
  uint16_t *out_lo;  // bf16 residual (or null)
  uint16_t *out_h16; // fp16 rounding of the result (or null)
  float *out_f32;    // fp32 result (or null)
  const int32_t *rows = nullptr;  // pooled row i is x row rows[i] (or i)
  int64_t in_stride = kBlk;       // rows of x between the first rows of blocks
  int64_t out_stride = 1;         // output rows between consecutive blocks
  int32_t *status = nullptr;      // workspace status word: kStatusRange on an fp16 overflow
  // PackedTile chunks [n_heads][n_cch] (or null): the fp16 result also goes
  // straight into the K rows (packed_v 0) or the V^T rows (packed_v 1) of
  // the chunk holding its block; rows past n_blk are zeroed
  uint16_t *packed = nullptr;
  int n_cch = 0, packed_v = 0;
};

struct CmpAttnParams {
  const uint16_t *q, *q_lo;    // [N, Hq, d] bf16; q_lo only for split operands
  const uint16_t *kc, *kc_lo;  // [n_blk, Hkv, d]: fp16, or bf16 hi/lo when split
  const uint16_t *vc;          // [n_blk, Hkv, d] fp16
  const uint16_t *kvc;         // packed tiles [Hkv][n_cch][K, V^T] (fp16 path), or null
  int n_cch;                   // chunks of 64 compressed blocks in kvc
  const float *gates;      // [N, Hq, 3]
  float *out;              // [N, Hq, d]
  float *lse;              // [n_vis, Hq]
  float *gs;               // frame-packed group scores
  int64_t v0;              // first vision position
  int n_vis, hq, hkv, n_frames;
  float sl2;               // softmax scale * log2(e)
  const int32_t *vmap = nullptr;  // vision row -> position (several vision runs)
  int32_t *status = nullptr;  // workspace status word (kStatusRange)
};

struct TopkParams {
  const float *gs;
  int32_t *sel;            // [n_vis, Hkv, k]
  int n_vis, hkv, k;
};

struct SwaParams {
  const uint16_t *q;           // [N, Hq, d]: bf16, or fp16
  const uint16_t *kv;          // packed vision blocks [Hkv][n_tiles][K, V^T]
  const float *gates;
  float *out;
  int64_t v0;
  int n_vis, hq, hkv, window, n_tiles;
  float sl2;
  const int32_t *vmap = nullptr;
};

struct SelParams {
  const uint16_t *q, *k, *v;
  uint16_t *kv;            // workspace: packed [Hkv][n_frames][K tile, V^T tile]
  const int32_t *sel;      // [n_vis, Hkv, k]
  const float *gates;
  float *out;
  int64_t v0;
  int n_vis, hq, hkv, topk, n_frames;
  float sl2;
  const int32_t *vmap = nullptr;
  int spin_limit = 1 << 22;      // bounded-wait rounds before a wave gives up
  int32_t *status = nullptr;     // workspace status word (kStatusWaitGaveUp on give-up)
};

struct TextParams {
  const uint16_t *q;       // [N, Hq, d]
  const uint16_t *kv_vis;  // packed vision blocks [Hkv][n_vchunks][K, V^T]
  const uint16_t *kv_txt;  // packed text rows [Hkv][n_tchunks][K, V^T]
  float *part_o;           // [n_split, n_text, Hq, d]
  float2 *part_ml;         // [n_split, n_text, Hq] (lse in log2 units, unused)
  float *out;              // merge target [N, Hq, d]
  int64_t v0, v1, n_tokens;
  int n_text, hq, hkv, n_split, chunks_per_split, n_tiles, n_vchunks, n_tchunks;
  float sl2;
  const int32_t *tmap = nullptr;  // text row -> position (several vision runs)
  const int32_t *tnvb = nullptr;  // text row -> vision tokens before it
};

struct DenseParams {
  const uint16_t *q;       // [N, Hq, d]: bf16, or fp16
  const uint16_t *kv;      // packed rows [Hkv][n_tiles][K, V^T]
  float *out;              // [N, Hq, d]
  float *lse;              // [N, Hq] natural log, or null
  int64_t n;               // tokens
  int hq, hkv, n_tiles;
  float sl2;
};

struct GateParams {
  const uint16_t *x;       // [N, d_model] bf16 hidden states
  const uint16_t *w1;      // [d_hidden, d_model] bf16
  const float *b1;         // [d_hidden] or null
  const uint16_t *w2;      // [3 Hq, d_hidden] bf16
  const float *b2;         // [3 Hq] or null
  uint16_t *h;             // workspace [N, d_hidden] fp16
  float *logits;           // [N, Hq, 3]
  int64_t n;
  int d_model, d_hidden, hq, act;  // act: 0 SiLU, 1 GELU (tanh form), 2 ReLU
};

struct BwdParams {
  const uint16_t *q, *k, *v, *wk, *wv;  // bf16: [N,Hq,d], [N,Hkv,d] x2, [d,d] x2
  const float *gates, *dout;            // [N,Hq,3], [N,Hq,d]
  const int32_t *sel;                   // [N_v,Hkv,k] selected blocks of the forward
  float *dq, *dk, *dv, *dgate, *dwk, *dwv;
  float *kc, *vc, *kbar, *vbar, *dkc, *dvc;  // workspace [n_blk,Hkv,d] each
  uint16_t *kc16, *vc16;                // workspace [n_blk,Hkv,d] fp16 compressed keys / values
  uint16_t *tile_v, *tile_p, *tile_c;   // backward tiles of the vision blocks, of all positions, of
                                        // the compressed keys: [Hkv][tiles][4 sections][64 d] fp16
  float *vstat;                         // [N_v,Hq,3,2]: per branch log2-sum-exp and dout . o
  float *tstat;                         // [N_t,Hq,2] the same for the text rows
  uint32_t *selmask;                    // [Hkv][n_vtile][mask_words]: bit t = vision token t chose it
  int32_t *selcnt, *seloff, *selrows;   // [Hkv n_vtile], [Hkv n_vtile + 1], [N_v Hkv k]: the tokens
                                        // that chose each (group, block), ascending
  float *cpart;                         // [n_ctile][n_chunk][Hkv][2][64][d] partial compressed grads
  float *tpart;                         // [n_tsplit][N_t Hq][d + 2] text rows' per-split partials
  int32_t *status;                      // the workspace's status word (bit 1: an fp16 range overflow)
  int spin_limit = 1 << 22;             // bounded-wait rounds of the query side's selection ring
  int64_t n, v0, n_vis;
  int hq, hkv, topk, window, n_blk;
  float scale;
  int n_vtile, n_ptile, n_ctile, mask_words, n_chunk, n_tsplit;
};

// One slice of the token-kind mask, as kernel arguments: bit j of word i
// says whether position base + 32 i + j is a vision token.
constexpr int kMaskWords = 512;
struct MaskSlice {
  uint32_t bits[kMaskWords];
  int64_t base;        // first position of the slice
  int64_t vis_before;  // vision tokens before `base`
  int n;               // positions in the slice (<= 32 * kMaskWords)
};

struct DecodeParams {
  const uint16_t *q;                // [Bt, Hq, d] bf16
  const uint16_t *kcache, *vcache;  // [Bt, L, Hkv, d] bf16
  const uint16_t *kc, *vc;          // [Bt, L/64, Hkv, d] bf16
  const float *gates;               // [Bt, Hq, 3]
  float *out;                       // [Bt, Hq, d]
  int32_t *sel;                     // [Bt, Hkv, k]
  float *lse;                       // [Bt, Hq] or null
  float *logits;                    // workspace [Bt, Hq, n_blk] scaled log2 logits
  float *cmp_part;                  // workspace [Bt, Hq, n_chunk, d + 2] (max, sum, o)
  float *ocmp;                      // workspace [Bt, Hq, d]
  float *fine_part;                 // workspace [Bt, Hq, n_items, d + 2]
  int batch, L, hq, hkv, topk, window, n_blk, n_chunk, n_win, n_items;
  int cap, cap_blk;  // cache rows and compressed rows per sequence (strides)
  int own;           // the query's own block, (L - 1) / 64 (= number of candidates)
  float sl2;
};

size_t pool_smem_bytes(int n_heads, int d);
hipError_t launch_cmp_pool(const PoolJob &j0, const PoolJob *j1, int d, bool fp32, hipStream_t st);
// The same pooling of two jobs (keys, values) as a block-mean launch into
// `means` (2 * n_blk * Hkv * d floats) and a map launch; identical results.
hipError_t launch_cmp_pool_split(const PoolJob &j0, const PoolJob &j1, int d, bool fp32, float *means,
                                 hipStream_t st);
// The map launch alone, over block means already in `means` (laid out as
// above; pack_kv with mean outputs writes them for bf16 layers).
hipError_t launch_cmp_map(const PoolJob &j0, const PoolJob &j1, int d, bool fp32, const float *means,
                          hipStream_t st);
// Copies one row of n_cols bf16 per sequence (src [Bt, n_cols]) to row `row`
// of dst [Bt, cap, n_cols], for keys and values at once.
hipError_t launch_append_rows(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_cache,
                              uint16_t *v_cache, int batch, int n_cols, int64_t cap, int64_t row,
                              hipStream_t st);
// fp32 -> bf16 high part (+ optional bf16 residual), or fp32 -> fp16.
hipError_t launch_split_bf16(const float *x, int64_t n, uint16_t *hi, uint16_t *lo, hipStream_t st);
hipError_t launch_to_f16(const float *x, int64_t n, uint16_t *out, hipStream_t st, int32_t *status = nullptr);
hipError_t launch_cmp_attn(const CmpAttnParams &p, int d, int G, bool split, hipStream_t st);
hipError_t launch_topk(const TopkParams &p, int n_blk_max, hipStream_t st);
// f16: q, k, v hold fp16 (else bf16; values are converted while staging)
hipError_t launch_swa_attn(const SwaParams &p, int d, int G, bool f16, hipStream_t st);
// mk, mv (or null): the column means of each complete block's keys and
// values ([n_mean][Hkv][d] floats, the pooling's block means, bitwise), taken
// from the bf16 rows as they are packed.
hipError_t launch_pack_kv(const SelParams &p, int d, bool f16, hipStream_t st, float *mk = nullptr,
                          float *mv = nullptr, int64_t n_mean = 0);
// Packs n_rows rows of k, v ([rows][Hkv][d]) into PackedTile blocks
// [Hkv][n_chunks][K tile, V^T tile]: packed row i is source row rows[i] when
// a map is given, else row0 + i, plus `jump` for i >= split_at; v_f16: v is
// fp16 already (else bf16, converted).
hipError_t launch_pack_tiles(const uint16_t *k, const uint16_t *v, int64_t row0, int n_rows, int hkv,
                             int n_chunks, uint16_t *out, int d, bool v_f16, hipStream_t st,
                             int split_at = 0x7fffffff, int64_t jump = 0,
                             const int32_t *rows = nullptr, int32_t *status = nullptr,
                             float *mk = nullptr, float *mv = nullptr, int64_t n_mean = 0);
// Writes the row maps of one mask slice: vmap[t] = position of vision row t,
// tmap[r] = position of text row r, tnvb[r] = vision tokens before it.
hipError_t launch_row_maps(const MaskSlice &m, int32_t *vmap, int32_t *tmap, int32_t *tnvb,
                           hipStream_t st);
size_t packed_kv_block_elems(int d);  // elements of one packed (K, V^T) block
hipError_t launch_sel_attn(const SelParams &p, int d, int G, bool f16, hipStream_t st);
// Sets the workspace status word to zero (a one-thread kernel, so the call
// stays free of memset nodes when captured into a graph).
hipError_t launch_status_clear(int32_t *status, hipStream_t st);
constexpr int32_t kStatusWaitGaveUp = 1;  // a bounded wait ran out: outputs are NaN
constexpr int32_t kStatusRange = 2;       // a value the kernels use in fp16 overflowed fp16's range
hipError_t launch_text_attn(const TextParams &p, int d, int G, bool f16, hipStream_t st);
hipError_t launch_text_merge(const TextParams &p, int d, hipStream_t st);
hipError_t launch_dense_attn(const DenseParams &p, int d, int G, bool f16, hipStream_t st);
// layer 0: hidden layer into p.h; layer 1: logits from p.h
hipError_t launch_gate(const GateParams &p, int layer, hipStream_t st);
// stage 0: clear accumulators; 1: pooling; 2: per-row gradients; 3: compression maps
hipError_t launch_backward(const BwdParams &p, int d, int stage, hipStream_t st);
hipError_t launch_decode(const DecodeParams &p, int d, int G, hipStream_t st);

// Which (head_dim, query heads per KV head) pairs have kernels.
bool supported_heads(int d, int G, bool split);
bool decode_supported(int d, int G);

}  // namespace nsa
