// Host-side launch interface of the device operations. Each launcher enqueues
// one kernel on `st`; shapes are validated by the caller (rlt_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

enum class Dt : int { F32 = 0, BF16 = 1, F16 = 2 };

// Row m of a logical [rows, width] matrix lives at  base + (m / tn) * sb + (m % tn) * st
// (elements). Covers contiguous buffers (tn = rows) and [B][Tmax][d] position slices.
struct RowMap {
  int64_t sb = 0, st = 0;
  int tn = 1;
  const int* pos = nullptr;   // per-sequence position offsets (device): + pos[m / tn] * pst
  int64_t pst = 0;
  __device__ int64_t off(int m) const {
    return (int64_t)(m / tn) * sb + (int64_t)(m % tn) * st + (pos ? (int64_t)pos[m / tn] * pst : 0);
  }
};
inline RowMap contiguous(int width) { RowMap r; r.tn = 1; r.sb = width; r.st = 0; return r; }

// Destination of keys/values: [B][H][cap][dh] blocks starting at k / v.
// Position p (1-based) of sequence b goes to slot (p - 1) % cap when ring != 0, else p - 1.
struct KVDst {
  void* k = nullptr;
  void* v = nullptr;
  int cap = 0;
  int ring = 0;
  int64_t lo = 0;   // > 0: two-term keys/values, the lo term of an element `lo` elements after its hi term
};

enum class Ep : int {
  StoreAct = 0,   // out[m*ldo + n] = act(acc)
  StoreF32,       // outf[m*ldo + n] = acc
  Residual,       // resid[rmap(m) + n] += acc
  SwiGLU,         // rows (2j, 2j+1) = (W1 x, W3 x): out[m*ldo + j] = act(silu(a) * b)
  QKV,            // n < hd: q = rope(acc) -> out; hd <= n < 2hd: k = rope -> kv.k; else v -> kv.v
                  // (two-term q when out_split > 0, two-term k / v when kv.lo > 0)
  RopeQ,          // out[m*ldo + n] = act(rope(acc))      (cross-attention query)
  MemKV,          // n < hd: k = rope -> kv.k; else v -> kv.v
  Merge,          // rows (2n, 2n+1) = (W_g,r r, W_s r): u = e + alpha*sigmoid(gpre + a)*b -> z
  Bias,           // outf[rmap(m) + n] = acc + bias[n]    (gate pre-activation W_g,e e + b_g)
};

struct EpArgs {
  void* out = nullptr;        // activation output (act type) or fp32 output for StoreF32
  int64_t ldo = 0;
  float* resid = nullptr;     // Residual: fp32 rows via rmap; Bias: fp32 out via rmap; Merge: z rows
  RowMap rmap;
  const float2* rope = nullptr;  // [pos][dh/2] (cos, sin), pos 0-based index = position
  int H = 0, dh = 0, hd = 0;
  int tn = 1;                 // rows per sequence in this GEMM: m -> b = m / tn, i = m % tn
  int pos0 = 0;               // position of i = 0 is pos0 + 1
  int b0 = 0;                 // sequence offset of row b = 0 inside the state
  KVDst kv;
  // Merge: e and gpre rows of (b, i) at rmap-like offsets eb * b + et * i; nrep outputs per row
  const float* e = nullptr;
  const float* gpre = nullptr;
  int64_t eb = 0, et = 0;
  int nrep = 1;
  float alpha = 0.f;
  const float* bias = nullptr;
  // Folded RMSNorm, producer side (Residual epilogue, decode GEMM): besides z += acc, write
  // fold_zb[m * fold_ld + n] = act(z_new * fold_gain[n]) and fold_ssp[m * (N / 16) + n / 16] =
  // sum of z_new^2 over the 16 features of the tile.
  // The Merge epilogue folds the same way (one row per sequence, nrep 1): fold_zb gets
  // act(u * fold_gain) and fold_ssp[m * (N / 16) + tile] the sum of u^2 over the tile's 8
  // features (N = 2d weight rows, so d / 8 partials per row).
  void* fold_zb = nullptr;
  float* fold_ssp = nullptr;
  const float* fold_gain = nullptr;
  int64_t fold_ld = 0;
  // Folded RMSNorm, consumer side (decode GEMM): acc of row m is scaled by
  // 1 / sqrt(sum_k rs_ssp[m * rs_n + k] / rs_d + rs_eps) before the epilogue, so X may hold
  // act(z * gain) instead of act(rms(z) * gain). rs_n a multiple of 4, <= 256.
  const float* rs_ssp = nullptr;
  int rs_n = 0;
  int rs_d = 0;
  float rs_eps = 0.f;
  // Two-term activations (16-bit types). out_split > 0: the SwiGLU output and the folded zb are
  // written as hi at their column and lo = v - hi at column + out_split. x_split != 0: each X row
  // holds K hi terms followed by K lo terms (row stride >= 2K) and the GEMM adds both products.
  int64_t out_split = 0;
  int x_split = 0;
  // Position from device memory (graph replay of a scan pass): when set, the pass's first
  // position index is pos_dev[0] instead of pos0, and the merge's e / gpre rows move by
  // pos_dev[0] * pos_stride elements.
  const int* pos_dev = nullptr;
  int64_t pos_stride = 0;
  // Per-sequence positions (rows at different positions, device memory): sequence b = m / tn of
  // this call has its first position index at row_pos[b] (overrides pos0 / pos_dev); the
  // merge's e / gpre rows of sequence b move by row_pos[b] * pos_stride elements.
  const int* row_pos = nullptr;
  // Copies of the new residual rows (Residual epilogue): dup_rows[dup_map.off(m) + n], and for
  // the last row of each sequence (m % tn == tn - 1) dup_last[(m / tn) * dup_last_ld + n].
  float* dup_rows = nullptr;
  RowMap dup_map;
  float* dup_last = nullptr;
  int64_t dup_last_ld = 0;
  // Row-invariant arithmetic: every row count takes the decode kernel, whose per-row sums
  // run in the same order whatever M is (a row's result does not depend on the batch).
  int row_invariant = 0;
  // The model's weights exceed the last-level cache: decode GEMMs of one row block load them
  // with the nontemporal hint.
  int stream_w = 0;
  // Split-K workspace of the decode GEMM (one launch at a time per workspace): the partial
  // 16x16 tiles of every K split ([split][row block][tile group][tile][lane] f32x4). Without
  // it (kpart null) every launch runs unsplit.
  float* kpart = nullptr;
  int64_t kpart_n = 0;        // floats
  // Decode tile shape forced by the caller (TPW, NMB, K splits; TPW 0: the cost model's choice),
  // taken where the shape admits it.
  int tile_ov[3] = {0, 0, 1};
};

// Largest row count the decode GEMM takes; folded RMSNorm is available up to it.
constexpr int kSkinnyMaxRows = 512;
// Most K splits of a decode GEMM.
constexpr int kMaxKSplit = 4;

// GEMM: Y[m, n] = sum_k X[m, k] * W[n, k]  (X act rows with leading dim ldx; W packed [N, K]:
// tile-major for bf16, row-major for fp32), Y consumed by the epilogue. bf16: MFMA; fp32:
// vector FMA.
void gemm(Dt dt, Ep ep, const EpArgs& a, const void* X, int64_t ldx, const void* W, int M, int N, int K,
          hipStream_t st);

// out[m, :] = act(rms(x[rmap(m), :]) * gain)  (gain may be null: plain cast); out_split > 0
// also writes the lo terms at column + out_split (two-term activations)
void rmsnorm(Dt dt, const float* x, RowMap xm, const float* gain, void* out, int64_t ldo, int rows, int d,
             float eps, hipStream_t st, int64_t out_split = 0);
// h[rmap(m), :] = emb[tok[m], :]  (fp32 out)
void embed(Dt dt, const int32_t* tok, const void* emb, float* h, RowMap hm, int rows, int d, hipStream_t st);
// rope table [npos][dh/2] (cos, sin) of angle p * base^(-2i/dh), evaluated in double precision
void rope_table(float2* tab, int npos, int dh, float base, hipStream_t st);
// dst[rmap_d(m), :] = src[rmap_s(m), :] (fp32 rows)
void copy_rows(const float* src, RowMap sm, float* dst, RowMap dm, int rows, int d, hipStream_t st);
// dst[rmap_d(m) + col * col_stride, :] = src[rmap_s(m), :] with col = col_dev[0] read on the device
void copy_rows_at(const float* src, RowMap sm, float* dst, RowMap dm, const int* col_dev, int64_t col_stride,
                  int rows, int d, hipStream_t st);
// scan position words for graph replay: p[0] = position index, p[1] = readout buffer column
void set_scan_pos(int* p, int pos, int col, hipStream_t st);
void advance_scan_pos(int* p, int np, hipStream_t st);
// *out_dev = order-independent 64-bit digest of n_words 64-bit words at p (device)
void digest64(const void* p, int64_t n_words, uint64_t* out_dev, hipStream_t st);
// p[0 .. n) = 0 (32-bit words), a kernel rather than a memset so the call is capture-safe
void fill_zero_u32(void* p, int64_t n, hipStream_t st);
// s[b, :] = s0 (fp32) for b < B; used for H_0 and the RLT-2 register
void broadcast_row(const float* s0, float* s, int B, int d, hipStream_t st);
// dst[b] <- src[b * src_ld ...] (src_ld 0: one vector for every row) where mask[b] != 0
void masked_rows(const float* src, int64_t src_ld, float* dst, const int* mask, int B, int d, hipStream_t st);
// out[b] = keep[b] ? 0 : tok[b]
void active_tokens(const int32_t* tok, const int* keep, int32_t* out, int B, hipStream_t st);
// out[om(r)] = L[tok[tm(r)]] - logsumexp(L) with L = logits row lm(r); tok < 0 writes 0
void logprob(const float* logits, RowMap lm, const int32_t* tok, RowMap tm, float* out, RowMap om, int rows,
             int V, hipStream_t st);
// Behaviour sampling (one workgroup per row): tok[b * tok_ld] = a draw from
// softmax(logits[b] / temperature) by Gumbel-max with Philox4x64-10 uniforms (key (seed, 0),
// counter (j / 4, b, step, 0)); lp[b * lp_ld] (nullable) = log of its probability;
// next[b] (nullable) = the token again. temperature 0: greedy, lp = 0.
void sample_rows(const float* logits, int64_t ld, int rows, int V, float temperature, uint64_t seed, uint64_t step,
                 int32_t* tok, int64_t tok_ld, float* lp, int64_t lp_ld, int32_t* next, hipStream_t st,
                 void* ws = nullptr);
// bytes of the optional sample_rows workspace (chunk statistics of every row) for rows x V
int64_t sample_workspace_bytes(int rows, int V);
// Size of the sampler's static scratch array (one per GPU, held until the process ends) and the
// current device's address of it (looked up once per device; no allocation).
constexpr int64_t kSampleScratchBytes = 1 << 20;
hipError_t sample_scratch(void** out);
// ratio[i] = exp(lp_cur[i] - lp_beh[i]) (float64 inside)
void importance_ratio(const float* lp_cur, const float* lp_beh, int64_t n, float* ratio, hipStream_t st);
// pack fp32 [N, K] into the library layout: dst row r <- src row perm(r); perm per kind.
// tiles = false: row-major [N][K] (dst_ld = K). tiles = true (bf16 GEMM weights): the
// tile-major layout below, with K = dst_ld a multiple of 64 and dst_col0 = 0.
//
// Tile-major bf16 weight layout. Rows are grouped in 16-row tiles (N padded to a multiple
// of 16); tile t occupies 16 * K contiguous elements made of K / 64 blocks of 1024 elements,
// one per 64-wide k chunk. Inside block c, element (row 16 t + r, k = 64 c + 16 g + 8 h + e)
// sits at 512 h + 8 (16 g + r) + e. Lane l = 16 g + r of a wavefront then finds the MFMA
// operand halves of its row r and k group g at l * 8 and 512 + l * 8: each load instruction
// of a wavefront reads 1 KB of contiguous memory.
enum class Pack : int { Plain = 0, RopeRows, Interleave2 };
void pack_matrix(Dt dt, const float* src, int64_t src_ld, int64_t col0, void* dst, int64_t dst_ld,
                 int64_t dst_col0, int rows, int cols, Pack kind, int dh, int row_stride, int row_off,
                 bool tiles, hipStream_t st);
// element offset of (row n, column k) in the tile-major layout of a [*, K] weight
__host__ __device__ inline int64_t tile_major_off(int64_t n, int64_t k, int64_t K) {
  const int64_t kk = k & 63;
  return (n >> 4) * 16 * K + (k >> 6) * 1024 + ((kk >> 3) & 1) * 512 + ((kk >> 4) * 16 + (n & 15)) * 8 + (kk & 7);
}

// Blocks of a key-split decode attention launch at most; a split workspace holds
// kAttnSplitBlocks * (dh + 2) floats.
constexpr int kAttnSplitBlocks = 2048;

// Attention of nq query rows per (sequence, head) over a position range of a key/value store.
struct AttnArgs {
  const void* q = nullptr;      // act [B*nq][H*dh] (roped, pairs interleaved like the keys)
  int64_t ldq = 0;
  const void* k = nullptr;      // [B][H][cap][dh] starting at b = 0 of this call
  const void* v = nullptr;
  int64_t kv_bstride = 0;       // elements between sequences
  int cap = 0;
  int ring = 0;                 // slot(p) = (p-1) % cap if ring else p-1
  void* out = nullptr;          // act [B*nq][H*dh]
  int64_t ldo = 0;
  int B = 0, nq = 1, H = 0, dh = 0;
  int pos0 = 0;                 // query i sits at position pos0 + 1 + i
  int window = 0;               // >0: keys max(1, p-window+1)..p ; 0: keys 1..p
  float scale = 1.f;
  int64_t out_split = 0;        // > 0: output lo terms at column + out_split (two-term activations)
  const int* pos_dev = nullptr; // when set, pos0 is read from pos_dev[0] (graph replay)
  const int* row_pos = nullptr; // when set, sequence b's pos0 is row_pos[b] (rows at different positions)
  // Key splits (load balance of few long key ranges; attn_decode only): split_ws holds
  // kAttnSplitBlocks * (dh + 2) floats, n_max bounds every query's key count (0: unknown, no
  // split), split_max caps the pieces per range. split_keys is set by the launcher.
  float* split_ws = nullptr;
  int split_max = 0;
  int n_max = 0;
  int split_keys = 0;
  // Two-term operands (16-bit types): q_lo > 0: each query row holds its lo terms q_lo elements
  // after the hi terms; kv_lo > 0: the lo term of a key / value element lies kv_lo elements after
  // its hi term. Scores and weighted sums then use (hi + lo) in fp32 (decode) or three MFMA
  // products hi*hi + hi*lo + lo*hi (prefill, whose probabilities are split the same way).
  int64_t q_lo = 0;
  int64_t kv_lo = 0;
  int stream = 0;               // 1: nontemporal key / value loads (the launch streams more than the
                                // last-level cache holds)
  int memory = 0;               // 1: the decoder's cross-attention over the memory (its own kernel
                                // instance, so profiles report it apart from the window attention)
  int wide = 0;                 // 1: a launch with no more blocks than CUs may take blocks of 512
                                // threads (a row's summation order then depends on the launch size:
                                // unset in batch-invariant mode)
};
void attn_decode(Dt dt, const AttnArgs& a, hipStream_t st);
// 16-bit many-query attention with MFMA (dh 64 or 128); returns false when the type or shape is
// not covered
bool attn_prefill(Dt dt, const AttnArgs& a, hipStream_t st);

}  // namespace rlt
