// C ABI of the RLT transition library: validation, weight packing, state
// ownership, and the launch schedules of encode / decode scan / step / replay.
//
// Sources: greeksharifa.github.io "Recurrent Looped Transformer 요약 설명"
// (§2.1-§2.7, appendix A.1, E, F, I) and jiphyeonjeon.kr "Recurrent Looped
// Transformer" (§2 eq 2.1-2.2, §3.1-§3.4 eq 2.7-2.16, §4.2 eq 3.3, §6.2 eq 5.5).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <stdexcept>
#include <string>
#include <vector>

#include "rlt.h"
#include "ops.hpp"
#include "scan.hpp"
#include "grad.hpp"

using namespace rlt;

namespace {

thread_local std::string g_err;

struct Fail {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, const std::string& msg) { throw Fail{code, msg}; }

#define HIPCHK(expr)                                                                        \
  do {                                                                                      \
    hipError_t _e = (expr);                                                                 \
    if (_e != hipSuccess) fail(RLT_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

template <typename F>
int guarded(F&& f) {
  try {
    f();
    return RLT_OK;
  } catch (const Fail& e) {
    g_err = e.msg;
    return e.code;
  } catch (const std::exception& e) {
    g_err = e.what();
    return RLT_ERR_INVALID_ARG;
  } catch (...) {
    g_err = "unknown error";
    return RLT_ERR_INVALID_ARG;
  }
}

void check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) fail(RLT_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
}

constexpr int kReadoutPositions = 64;   // positions per batched readout
constexpr int kMaxSlices = 4;           // concurrent batch slices of the launch-path scan
constexpr int kParallelPositions = 64;  // RLT-0 positions per decoder pass
constexpr int64_t kEncoderRows = 32768; // encoder workspace rows (sequences x tokens per group)
constexpr int64_t kStreamBytes = 256ll << 20;   // last-level cache: larger streams load nontemporally
constexpr int kStage = 8;               // pinned staging slots of the per-row position arrays

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct LayerW {
  float *n1 = nullptr, *n2 = nullptr, *n3 = nullptr;  // enc: n1, n2; dec: m1, m2, m3
  void *wqkv = nullptr, *wo = nullptr, *w13 = nullptr, *w2 = nullptr;
  void *xq = nullptr, *xo = nullptr;
};

}  // namespace

struct rlt_model {
  rlt_config cfg{};
  int device = 0;
  Dt dt = Dt::BF16;
  size_t esz = 2;
  int act = 1;   // 2: GEMM activation inputs are two-term (hi | lo) 16-bit rows
  int hd = 0;
  void* arena = nullptr;
  size_t arena_bytes = 0;
  void* emb = nullptr;
  std::vector<LayerW> enc, dec;
  float* nE = nullptr;
  std::vector<void*> wkv;
  float *ns = nullptr, *bg = nullptr, *s0 = nullptr;
  void *wg_e = nullptr, *wsr = nullptr;
  float* nO = nullptr;
  void* wout = nullptr;
  uint64_t version = 1;
  uint64_t wdigest = 0;   // digest of the packed parameter values (identifies a snapshot's weights)
  int scan_mode = 0;
  int batch_invariant = 0;   // every kernel's per-row arithmetic independent of batch and pass shape
  int tile_ov[3] = {0, 0, 1};   // decode GEMM tile override (TPW, NMB, K splits) from RLT_SKINNY_TILE
  int n_states = 0;
  // kernel timers (measurement): launches of each kind bracketed by events on their stream
  bool timing = false;
  std::vector<hipEvent_t> ev_free;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> timed[RLT_TIME_KINDS];
};

struct rlt_state {
  rlt_model* m = nullptr;
  int B = 0, Tm = 0, keep_enc = 0;   // Tm: position pitch of every per-position store (max_len + 1)
  int cap = 0;                        // max_len: positions a sequence may hold
  int P = 1;          // max positions per decoder pass
  int R = 1;          // ring capacity (slots per layer, sequence, head)
  int n_enc = 0, n_dec = 0;
  uint64_t version = 0;
  int64_t block_steps = 0;
  int64_t bytes[6] = {0, 0, 0, 0, 0, 0};
  std::vector<void*> allocs;
  float *s = nullptr, *rho = nullptr;
  float *e = nullptr, *gpre = nullptr;   // [B][Tm][d]
  void *mem_k = nullptr, *mem_v = nullptr;   // [G][B][H][Tm][dh]
  void *enc_k = nullptr, *enc_v = nullptr;   // [term][L_E][B][H][Tm][dh] (one term, or hi and lo planes)
  int64_t enc_lo = 0;                        // elements from a C^E hi term to its lo term (0: one term)
  int64_t ekv_lo = 0;                        // the same for ekv_k / ekv_v
  void *ring_k = nullptr, *ring_v = nullptr; // [L_D][B][H][R][dh]
  float2* rope = nullptr;                    // [Tm + 1][dh / 2]
  // decoder workspace, rows = B * P
  float* z = nullptr;
  void *xa = nullptr, *q = nullptr, *ao = nullptr, *hid = nullptr;
  float* dssp = nullptr;   // [rows][d / 8] partial sums of squares of z (folded RMSNorm)
  void* xs = nullptr;      // [B][act d] merge input: RMSNorm_s(s), or s * gain folded by the last block
  float* sssp = nullptr;   // [B][d / 16] partial sums of squares of s (folded merge input)
  // readout workspace, rows = B * kReadoutPositions
  float* sbuf = nullptr;
  void* xr = nullptr;
  float* lbuf = nullptr;
  // encoder workspace, rows = enc_rows
  int64_t enc_rows = 0;
  void *exa = nullptr, *eq = nullptr, *eao = nullptr, *ehid = nullptr;
  void *ekv_k = nullptr, *ekv_v = nullptr;   // attention keys when no encoder cache is kept
  int32_t* toks = nullptr;                   // [B][Tm] shifted next tokens (replay)
  float* glog = nullptr;                     // [B][V] logits of a generation step
  int32_t* gtok = nullptr;                   // [B] token drawn last, consumed by the next step
  float* lp = nullptr;                       // [B][Tm] log-probabilities (replay)
  // persistent scan (bf16 configurations it supports)
  bool scan_ok = false;
  float* pz[2] = {nullptr, nullptr};
  void* pzb[2] = {nullptr, nullptr};
  float* pssp[2] = {nullptr, nullptr};
  void *pq = nullptr, *pao = nullptr, *phid = nullptr, *rhob = nullptr;
  float* rhoss = nullptr;
  float* sall = nullptr;                     // [B][Tm][d] s_t of every position
  unsigned* bar = nullptr;
  rlt::ScanLayer* layers_dev = nullptr;
  int* abort_host = nullptr;                 // pinned copy of the scan's abort word
  int scan_grid = 0;
  // launch-path scan: batch slices run as independent chains on their own streams
  hipStream_t sub[kMaxSlices] = {};
  hipEvent_t ev_fork = nullptr;
  hipEvent_t ev_join[kMaxSlices] = {};
  // graph replay of one RLT-1 position (launch path): [0] without, [1] with readout rows
  int* pos_dev = nullptr;                    // [0] position index of the pass, [1] readout column
  // [with readout rows][merge input folded by the previous replay]
  hipGraphExec_t pass_graph[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
  // rows at different positions (rlt_step_rows / rlt_state_reset_rows)
  bool ragged = false;
  std::vector<int> row_n;             // positions consumed by each row (while ragged)
  int* rp_dev = nullptr;              // [3][B]: position index, row stays, register update
  int32_t* rtok = nullptr;            // [B] tokens of the rows that move
  float* s_bak = nullptr;             // [B][d] s before a per-row step
  float* attn_ws = nullptr;           // [kMaxSlices][kAttnSplitBlocks][dh + 2] key-split partials
  float* kpart = nullptr;             // [kMaxSlices][kpart_slice] split-K partial tiles of decode GEMMs
  int64_t kpart_slice = 0;
  void* samp_ws = nullptr;            // chunk statistics of the generation sampler
  int* rp_host = nullptr;             // pinned [kStage][3][B] staging of rp_dev
  hipEvent_t rp_ev[kStage] = {};
  bool rp_used[kStage] = {};
  int rp_next = 0;
};

namespace {

// `logical` (when >= 0) is the part reported under cls; the rest counts as workspace (class 5).
void* dev_alloc(rlt_state* s, size_t bytes, int cls, int64_t logical = -1) {
  void* p = nullptr;
  if (bytes == 0) return nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) fail(RLT_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  s->allocs.push_back(p);
  const int64_t rep = logical >= 0 ? logical : (int64_t)bytes;
  s->bytes[cls] += rep;
  s->bytes[5] += (int64_t)bytes - rep;
  return p;
}

void validate_config(const rlt_config& c) {
  auto bad = [](const std::string& m) { fail(RLT_ERR_INVALID_ARG, "config: " + m); };
  if (c.vocab <= 0 || c.vocab % 4) bad("vocab must be a positive multiple of 4");
  if (c.vocab > (1 << 20)) fail(RLT_ERR_UNSUPPORTED, "vocab > 2^20");
  if (c.d <= 0 || c.d % 64) bad("d must be a positive multiple of 64");
  if (c.n_heads <= 0 || c.d_head <= 0) bad("heads");
  if (c.d_head % 2) fail(RLT_ERR_UNSUPPORTED, "d_head must be even (rotary pairs)");
  if (c.d_head != 16 && c.d_head != 32 && c.d_head != 64 && c.d_head != 128 && c.d_head != 256)
    fail(RLT_ERR_UNSUPPORTED, "d_head must be 16, 32, 64, 128 or 256");
  if ((c.n_heads * c.d_head) % 64) bad("n_heads * d_head must be a multiple of 64");
  if (c.L_E < 1 || c.L_D < 0) bad("depths");
  if (c.ffn <= 0 || c.ffn % 64) bad("ffn must be a positive multiple of 64");
  if (c.window < 1) bad("window must be >= 1");
  if (c.L_D > 0 && !(c.groups == 1 || c.groups == c.L_D))
    fail(RLT_ERR_UNSUPPORTED, "memory groups must be 1 or L_D");
  if (c.variant != RLT_V0 && c.variant != RLT_V1 && c.variant != RLT_V2) bad("variant");
  if (c.chunk < 1 || (c.variant != RLT_V2 && c.chunk != 1)) bad("chunk must be 1 unless RLT-2");
  if (c.chunk > 64) fail(RLT_ERR_UNSUPPORTED, "chunk > 64");
  if (c.share_enc_dec && c.L_E != c.L_D) fail(RLT_ERR_UNSUPPORTED, "sharing needs L_E == L_D");
  if (c.dtype != RLT_FP32 && c.dtype != RLT_BF16 && c.dtype != RLT_FP16 && c.dtype != RLT_FP16X2) bad("dtype");
  if (!(c.rms_eps >= 0.f) || !(c.rope_base > 0.f)) bad("eps / rope base");
}

struct Shape {
  int64_t rows, cols;
};

std::map<std::string, Shape> manifest(const rlt_config& c) {
  std::map<std::string, Shape> m;
  const int64_t d = c.d, hd = (int64_t)c.n_heads * c.d_head, f = c.ffn, V = c.vocab;
  m["emb"] = {V, d};
  for (int l = 0; l < c.L_E; ++l) {
    const std::string p = "enc." + std::to_string(l) + ".";
    m[p + "n1"] = {1, d}; m[p + "n2"] = {1, d};
    m[p + "wq"] = {hd, d}; m[p + "wk"] = {hd, d}; m[p + "wv"] = {hd, d}; m[p + "wo"] = {d, hd};
    m[p + "w1"] = {f, d}; m[p + "w3"] = {f, d}; m[p + "w2"] = {d, f};
  }
  if (c.L_D > 0) {
    m["mem.nE"] = {1, d};
    for (int g = 0; g < c.groups; ++g) {
      m["mem." + std::to_string(g) + ".wk"] = {hd, d};
      m["mem." + std::to_string(g) + ".wv"] = {hd, d};
    }
  }
  if (c.variant != RLT_V0) {
    m["merge.ns"] = {1, d}; m["merge.wg"] = {d, 2 * d}; m["merge.bg"] = {1, d};
    m["merge.ws"] = {d, d}; m["merge.s0"] = {1, d};
  }
  for (int l = 0; l < c.L_D; ++l) {
    const std::string p = "dec." + std::to_string(l) + ".";
    m[p + "m1"] = {1, d}; m[p + "m2"] = {1, d}; m[p + "m3"] = {1, d};
    m[p + "xq"] = {hd, d}; m[p + "xo"] = {d, hd};
    if (!c.share_enc_dec) {
      m[p + "wq"] = {hd, d}; m[p + "wk"] = {hd, d}; m[p + "wv"] = {hd, d}; m[p + "wo"] = {d, hd};
      m[p + "w1"] = {f, d}; m[p + "w3"] = {f, d}; m[p + "w2"] = {d, f};
    }
  }
  m["out.nO"] = {1, d};
  m["out.w"] = {V, d};
  return m;
}

std::map<std::string, const float*> index_weights(const rlt_config& c, const rlt_tensor* w, int n) {
  if (n < 0 || (n > 0 && !w)) fail(RLT_ERR_INVALID_ARG, "weights pointer");
  auto man = manifest(c);
  std::map<std::string, const float*> got;
  for (int i = 0; i < n; ++i) {
    if (!w[i].name || !w[i].data) fail(RLT_ERR_INVALID_ARG, "null weight name or data");
    auto it = man.find(w[i].name);
    if (it == man.end()) fail(RLT_ERR_INVALID_ARG, std::string("unknown weight ") + w[i].name);
    if (w[i].numel != it->second.rows * it->second.cols)
      fail(RLT_ERR_INVALID_ARG, std::string("wrong size for ") + w[i].name);
    if (got.count(w[i].name)) fail(RLT_ERR_INVALID_ARG, std::string("duplicate weight ") + w[i].name);
    got[w[i].name] = w[i].data;
  }
  for (auto& kv : man)
    if (!got.count(kv.first)) fail(RLT_ERR_INVALID_ARG, "missing weight " + kv.first);
  return got;
}

// Lay out the packed parameter arena (sizes only) and assign pointers.
void layout_model(rlt_model* m, char* base, size_t* total) {
  const rlt_config& c = m->cfg;
  const size_t e = m->esz;
  const int64_t d = c.d, hd = m->hd, f = c.ffn, V = c.vocab;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  auto takef = [&](int64_t n) { return (float*)take(n * 4); };
  // GEMM weight [N, K]: bf16 weights hold whole 256-row groups of tiles (zero padding rows), the
  // unit the large-tile GEMM reads
  auto takew = [&](int64_t N, int64_t K) {
    const int64_t rows = m->dt != Dt::F32 ? (N + 255) / 256 * 256 : N;
    return take(rows * K * e);
  };
  m->emb = take(V * d * e);
  m->enc.assign(c.L_E, LayerW{});
  for (auto& L : m->enc) {
    L.n1 = takef(d); L.n2 = takef(d);
    L.wqkv = takew(3 * hd, d); L.wo = takew(d, hd); L.w13 = takew(2 * f, d); L.w2 = takew(d, f);
  }
  m->wkv.assign(c.L_D > 0 ? c.groups : 0, nullptr);
  if (c.L_D > 0) {
    m->nE = takef(d);
    for (auto& p : m->wkv) p = takew(2 * hd, d);
  }
  if (c.variant != RLT_V0) {
    m->ns = takef(d); m->bg = takef(d); m->s0 = takef(d);
    m->wg_e = takew(d, d); m->wsr = takew(2 * d, d);
  }
  m->dec.assign(c.L_D, LayerW{});
  for (int l = 0; l < c.L_D; ++l) {
    LayerW& L = m->dec[l];
    L.n1 = takef(d); L.n2 = takef(d); L.n3 = takef(d);
    L.xq = takew(hd, d); L.xo = takew(d, hd);
    if (c.share_enc_dec) {
      L.wqkv = m->enc[l].wqkv; L.wo = m->enc[l].wo; L.w13 = m->enc[l].w13; L.w2 = m->enc[l].w2;
    } else {
      L.wqkv = takew(3 * hd, d); L.wo = takew(d, hd); L.w13 = takew(2 * f, d); L.w2 = takew(d, f);
    }
  }
  m->nO = takef(d);
  m->wout = takew(V, d);
  *total = off;
}

void pack_all(rlt_model* m, const std::map<std::string, const float*>& W, hipStream_t st) {
  const rlt_config& c = m->cfg;
  const int d = c.d, hd = m->hd, f = c.ffn, V = c.vocab, dh = c.d_head;
  const Dt dt = m->dt;
  auto vec = [&](float* dst, const std::string& name) {
    HIPCHK(hipMemcpyAsync(dst, W.at(name), sizeof(float) * d, hipMemcpyDeviceToDevice, st));
  };
  const bool tiles = dt != Dt::F32;   // GEMM weights: tile-major in the 16-bit types
  auto plain = [&](void* dst, const std::string& name, int rows, int cols, int row_off = 0, int stride = 1) {
    pack_matrix(dt, W.at(name), cols, 0, dst, cols, 0, rows, cols, Pack::Plain, dh, stride, row_off, tiles, st);
  };
  auto roped = [&](void* dst, const std::string& name, int row_off) {
    pack_matrix(dt, W.at(name), d, 0, dst, d, 0, hd, d, Pack::RopeRows, dh, 1, row_off, tiles, st);
  };
  auto attn_ffn = [&](const LayerW& L, const std::string& p) {
    roped(L.wqkv, p + "wq", 0);
    roped(L.wqkv, p + "wk", hd);
    plain(L.wqkv, p + "wv", hd, d, 2 * hd);
    plain(L.wo, p + "wo", d, hd);
    plain(L.w13, p + "w1", f, d, 0, 2);   // SwiGLU pair rows (2j, 2j + 1) = (W1 row j, W3 row j)
    plain(L.w13, p + "w3", f, d, 1, 2);
    plain(L.w2, p + "w2", d, f);
  };
  // the embedding is gathered by rows, not a GEMM operand: row-major
  pack_matrix(dt, W.at("emb"), d, 0, m->emb, d, 0, V, d, Pack::Plain, dh, 1, 0, false, st);
  for (int l = 0; l < c.L_E; ++l) {
    const std::string p = "enc." + std::to_string(l) + ".";
    vec(m->enc[l].n1, p + "n1");
    vec(m->enc[l].n2, p + "n2");
    attn_ffn(m->enc[l], p);
  }
  if (c.L_D > 0) {
    vec(m->nE, "mem.nE");
    for (int g = 0; g < c.groups; ++g) {
      const std::string p = "mem." + std::to_string(g) + ".";
      roped(m->wkv[g], p + "wk", 0);
      plain(m->wkv[g], p + "wv", hd, d, hd);
    }
  }
  if (c.variant != RLT_V0) {
    vec(m->ns, "merge.ns");
    vec(m->bg, "merge.bg");
    vec(m->s0, "merge.s0");
    // W_g = [W_g,e | W_g,r] over [e_t ; r]: the e half is applied once per position at encode time,
    // the r half is interleaved with W_s (rows 2n, 2n + 1) for the per-step merge GEMM.
    pack_matrix(dt, W.at("merge.wg"), 2 * d, 0, m->wg_e, d, 0, d, d, Pack::Plain, dh, 1, 0, tiles, st);
    pack_matrix(dt, W.at("merge.wg"), 2 * d, d, m->wsr, d, 0, d, d, Pack::Plain, dh, 2, 0, tiles, st);
    pack_matrix(dt, W.at("merge.ws"), d, 0, m->wsr, d, 0, d, d, Pack::Plain, dh, 2, 1, tiles, st);
  }
  for (int l = 0; l < c.L_D; ++l) {
    const std::string p = "dec." + std::to_string(l) + ".";
    vec(m->dec[l].n1, p + "m1");
    vec(m->dec[l].n2, p + "m2");
    vec(m->dec[l].n3, p + "m3");
    pack_matrix(dt, W.at(p + "xq"), d, 0, m->dec[l].xq, d, 0, hd, d, Pack::RopeRows, dh, 1, 0, tiles, st);
    plain(m->dec[l].xo, p + "xo", d, hd);
    if (!c.share_enc_dec) attn_ffn(m->dec[l], p);
  }
  vec(m->nO, "out.nO");
  plain(m->wout, "out.w", V, d);
  check_launch();
}

// Digest of the packed parameters, computed on the device when they are set.
uint64_t weights_digest(rlt_model* m, hipStream_t st) {
  uint64_t* d = nullptr;
  if (hipMalloc((void**)&d, 16) != hipSuccess) fail(RLT_ERR_OOM, "digest scratch allocation failed");
  uint64_t h = 0;
  digest64(m->arena, (int64_t)(m->arena_bytes / 8), d, st);
  const hipError_t e1 = hipMemcpyAsync(&h, d, 8, hipMemcpyDeviceToHost, st);
  const hipError_t e2 = hipStreamSynchronize(st);
  (void)hipFree(d);
  if (e1 != hipSuccess || e2 != hipSuccess) fail(RLT_ERR_HIP, "weights digest failed");
  return h;
}

// FNV-1a over the configuration fields that shape the state
uint64_t config_digest(const rlt_config& c) {
  uint64_t h = 0xCBF29CE484222325ull;
  auto add = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= 0x100000001B3ull;
    }
  };
  uint32_t a, e, r;
  std::memcpy(&a, &c.alpha, 4);
  std::memcpy(&e, &c.rms_eps, 4);
  std::memcpy(&r, &c.rope_base, 4);
  for (uint64_t v : {(uint64_t)c.vocab, (uint64_t)c.d, (uint64_t)c.n_heads, (uint64_t)c.d_head, (uint64_t)c.L_E,
                     (uint64_t)c.L_D, (uint64_t)c.ffn, (uint64_t)c.window, (uint64_t)c.groups, (uint64_t)c.variant,
                     (uint64_t)c.chunk, (uint64_t)c.share_enc_dec, (uint64_t)c.dtype, (uint64_t)a, (uint64_t)e,
                     (uint64_t)r})
    add(v);
  return h;
}

void check_state(rlt_model* m, rlt_state* s) {
  if (!m || !s) fail(RLT_ERR_INVALID_ARG, "null model or state");
  if (s->m != m) fail(RLT_ERR_INVALID_ARG, "state belongs to another model");
  if (s->version != m->version) fail(RLT_ERR_STALE_STATE, "state was built under older weights; reset it");
  if (s->abort_host && *(volatile int*)s->abort_host)
    fail(RLT_ERR_HIP, "a persistent scan on this state timed out in a grid barrier; its results are invalid");
}

// GEMM of this model: the row-invariant dispatch when the model asks for batch-invariant
// arithmetic.
// Key-split workspace of a slice for attention launches whose key counts are at most n_max
// (none in batch-invariant mode: the split depends on the batch).
void attn_split(const rlt_model* m, const rlt_state* s, AttnArgs& at, int slice, int n_max) {
  if (m->batch_invariant || n_max <= 0) return;
  at.split_ws = s->attn_ws + (int64_t)slice * kAttnSplitBlocks * (m->cfg.d_head + 2);
  at.split_max = 64;
  at.n_max = n_max;
}


// Runs launch() and, while the model's timers are on and the stream is not being captured,
// brackets it with a pair of events recorded on that stream.
template <typename F>
void timed(rlt_model* m, int kind, hipStream_t st, F&& launch) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (!m->timing || hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    launch();
    return;
  }
  hipEvent_t ev[2];
  for (auto& e : ev) {
    if (m->ev_free.empty()) {
      HIPCHK(hipEventCreate(&e));
    } else {
      e = m->ev_free.back();
      m->ev_free.pop_back();
    }
  }
  HIPCHK(hipEventRecord(ev[0], st));
  launch();
  HIPCHK(hipEventRecord(ev[1], st));
  m->timed[kind].push_back({ev[0], ev[1]});
}

// slice: the concurrent batch slice the launch belongs to (its own split-K workspace)
void mgemm(rlt_model* m, rlt_state* s, int slice, int kind, Dt dt, Ep ep, EpArgs a, const void* X, int64_t ldx,
           const void* W, int M, int N, int K, hipStream_t st) {
  a.row_invariant = m->batch_invariant;
  a.tile_ov[0] = m->tile_ov[0];
  a.tile_ov[1] = m->tile_ov[1];
  a.tile_ov[2] = m->tile_ov[2];
  if (s->kpart) {
    a.kpart = s->kpart + (int64_t)slice * s->kpart_slice;
    a.kpart_n = s->kpart_slice;
  }
  a.stream_w = (int64_t)m->arena_bytes > kStreamBytes;
  timed(m, kind, st, [&] { gemm(dt, ep, a, X, ldx, W, M, N, K, st); });
}

// ------------------------------------------------------------------ encode
// row_pos (device [B], rows at different positions): sequence b encodes position row_pos[b] + 1
// (T = 1) instead of n_enc + 1 .. n_enc + T; the state's n_enc is then left to the caller.
void do_encode(rlt_model* m, rlt_state* s, const int32_t* tokens, int T, hipStream_t st,
               const int* row_pos = nullptr, int pos_max = 0) {
  const rlt_config& c = m->cfg;
  const Dt dt = m->dt;
  const int d = c.d, hd = m->hd, f = c.ffn, H = c.n_heads, dh = c.d_head, Tm = s->Tm;
  const int t0 = row_pos ? 0 : s->n_enc;
  const int Bc = (int)std::max<int64_t>(1, std::min<int64_t>(s->B, s->enc_rows / T));
  // GEMM activation rows: width w, or w hi terms then w lo terms (two-term activations)
  const int A = m->act, ad = A * d, ahd = A * hd, af = A * f;
  const int64_t sd = A > 1 ? d : 0, shd = A > 1 ? hd : 0, sf = A > 1 ? f : 0;
  for (int b0 = 0; b0 < s->B; b0 += Bc) {
    const int nb = std::min(Bc, s->B - b0);
    const int rows = nb * T;
    RowMap hm;   // encoder residual stream lives in the state's e rows
    hm.tn = T; hm.sb = (int64_t)Tm * d; hm.st = d;
    const int* rp = row_pos ? row_pos + b0 : nullptr;
    if (rp) { hm.pos = rp; hm.pst = d; }
    float* h = s->e + ((int64_t)b0 * Tm + t0) * d;
    embed(dt, tokens + (int64_t)b0 * T, m->emb, h, hm, rows, d, st);
    for (int l = 0; l < c.L_E; ++l) {
      const LayerW& L = m->enc[l];
      rmsnorm(dt, h, hm, L.n1, s->exa, ad, rows, d, c.rms_eps, st, sd);
      // q, k, v: two-term (hi, lo) with two-term GEMM inputs: q rows [hi | lo], keys and values
      // in a lo plane after the hi plane
      EpArgs a;
      a.out = s->eq; a.ldo = ahd; a.out_split = shd; a.rope = s->rope; a.H = H; a.dh = dh; a.hd = hd;
      a.tn = T; a.pos0 = t0; a.x_split = A > 1; a.row_pos = rp;
      AttnArgs at;
      at.row_pos = rp;
      at.wide = !m->batch_invariant;
      if (s->enc_k) {
        const int64_t lo = (int64_t)l * s->B * H * Tm * dh;
        a.kv.k = (char*)s->enc_k + lo * m->esz; a.kv.v = (char*)s->enc_v + lo * m->esz;
        a.kv.cap = Tm; a.b0 = b0; a.kv.lo = s->enc_lo;
        at.k = (char*)a.kv.k + (int64_t)b0 * H * Tm * dh * m->esz;
        at.v = (char*)a.kv.v + (int64_t)b0 * H * Tm * dh * m->esz;
        at.kv_bstride = (int64_t)H * Tm * dh; at.cap = Tm; at.kv_lo = s->enc_lo;
      } else {
        a.kv.k = s->ekv_k; a.kv.v = s->ekv_v; a.kv.cap = T; a.b0 = 0; a.kv.lo = s->ekv_lo;
        at.k = s->ekv_k; at.v = s->ekv_v; at.kv_bstride = (int64_t)H * T * dh; at.cap = T; at.kv_lo = s->ekv_lo;
      }
      a.kv.ring = 0;
      mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::QKV, a, s->exa, ad, L.wqkv, rows, 3 * hd, d, st);
      at.q = s->eq; at.ldq = ahd; at.q_lo = shd; at.ring = 0; at.out = s->eao; at.ldo = ahd; at.out_split = shd;
      at.B = nb; at.nq = T; at.H = H; at.dh = dh; at.pos0 = t0; at.window = 0;
      at.scale = 1.f / std::sqrt((float)dh);
      attn_split(m, s, at, 0, row_pos ? pos_max : t0 + T);
      timed(m, RLT_TIME_ENCODER_ATTN, st, [&] {
        if (!(T >= 16 && !m->batch_invariant && attn_prefill(dt, at, st))) attn_decode(dt, at, st);
      });
      EpArgs r; r.resid = h; r.rmap = hm; r.x_split = A > 1;
      mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::Residual, r, s->eao, ahd, L.wo, rows, d, hd, st);
      rmsnorm(dt, h, hm, L.n2, s->exa, ad, rows, d, c.rms_eps, st, sd);
      EpArgs sw; sw.out = s->ehid; sw.ldo = af; sw.out_split = sf; sw.x_split = A > 1;
      mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::SwiGLU, sw, s->exa, ad, L.w13, rows, 2 * f, d, st);
      mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::Residual, r, s->ehid, af, L.w2, rows, d, f, st);
    }
    if (c.L_D > 0) {
      // memory: k^g = RoPE(W^g_K RMSNorm_E(e)), v^g = W^g_V RMSNorm_E(e)  (eq 2.1-2.2)
      rmsnorm(dt, h, hm, m->nE, s->exa, ad, rows, d, c.rms_eps, st, sd);
      for (int g = 0; g < c.groups; ++g) {
        EpArgs a;
        a.rope = s->rope; a.H = H; a.dh = dh; a.hd = hd; a.tn = T; a.pos0 = t0; a.b0 = b0; a.row_pos = rp;
        const int64_t go = (int64_t)g * s->B * H * Tm * dh * m->esz;
        a.kv.k = (char*)s->mem_k + go; a.kv.v = (char*)s->mem_v + go; a.kv.cap = Tm; a.kv.ring = 0;
        a.x_split = A > 1;
        mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::MemKV, a, s->exa, ad, m->wkv[g], rows, 2 * hd, d, st);
      }
    }
    if (c.variant != RLT_V0) {
      // gate pre-activation W_g,e e_t + b_g: independent of the recurrence, computed token-parallel
      rmsnorm(dt, h, hm, nullptr, s->exa, ad, rows, d, 0.f, st, sd);
      EpArgs a; a.resid = s->gpre + ((int64_t)b0 * Tm + t0) * d; a.rmap = hm; a.bias = m->bg;
      a.x_split = A > 1;
      mgemm(m, s, 0, RLT_TIME_ENCODER_GEMM, dt, Ep::Bias, a, s->exa, ad, m->wg_e, rows, d, d, st);
    }
  }
  check_launch();
  if (!row_pos) s->n_enc += T;
}

// ------------------------------------------------------------------ decoder pass
// Positions t0+1 .. t0+np for every sequence, rows m = b * np + i.
// Sequences b0 .. b0+nb-1 of the state (a batch slice): the pointers of its rows.
struct SliceBufs {
  int b0 = 0, B = 0;
  int slice = 0;   // index of the concurrent slice (its own key-split workspace)
  float *z, *s, *rho, *e, *gpre, *dssp, *sssp;
  void *xa, *xs, *q, *ao, *hid, *ring_k, *ring_v, *mem_k, *mem_v;
};
SliceBufs slice_bufs(rlt_model* m, rlt_state* s, int b0, int nb) {
  const rlt_config& c = m->cfg;
  const int64_t d = c.d, hd = m->hd, f = c.ffn, P = s->P, e = m->esz;
  SliceBufs v;
  v.b0 = b0; v.B = nb;
  const int64_t r0 = (int64_t)b0 * P;   // first workspace row of the slice
  v.z = s->z + r0 * d; v.dssp = s->dssp + r0 * (d / 8);
  const int64_t A = m->act;
  v.xs = (char*)s->xs + (int64_t)b0 * A * d * e; v.sssp = s->sssp + (int64_t)b0 * (d / 16);
  v.xa = (char*)s->xa + r0 * A * d * e; v.q = (char*)s->q + r0 * hd * e;
  v.ao = (char*)s->ao + r0 * A * hd * e; v.hid = (char*)s->hid + r0 * A * f * e;
  v.s = s->s + (int64_t)b0 * d; v.rho = s->rho + (int64_t)b0 * d;
  v.e = s->e + (int64_t)b0 * s->Tm * d;
  v.gpre = s->gpre ? s->gpre + (int64_t)b0 * s->Tm * d : nullptr;
  const int64_t kvb = (int64_t)c.n_heads * c.d_head * e;   // bytes per position of one sequence
  v.ring_k = s->ring_k ? (char*)s->ring_k + (int64_t)b0 * s->R * kvb : nullptr;
  v.ring_v = s->ring_v ? (char*)s->ring_v + (int64_t)b0 * s->R * kvb : nullptr;
  v.mem_k = s->mem_k ? (char*)s->mem_k + (int64_t)b0 * s->Tm * kvb : nullptr;
  v.mem_v = s->mem_v ? (char*)s->mem_v + (int64_t)b0 * s->Tm * kvb : nullptr;
  return v;
}

// Links between consecutive passes of one scan call.
struct PassIO {
  bool in_folded = false;   // xs / sssp hold s_{t-1} * gain_s and its partial sums of squares,
                            // written by the previous pass's last block (RLT-1, folded norms)
  bool out_fold = false;    // this pass's last block writes them for the next pass
  float* rows = nullptr;    // this pass's output rows z also go to rows[rows_map.off(m)]
  RowMap rows_map;
};

// pos_dev (graph replay, RLT-1): positions come from pos_dev[0] on the device instead of t0.
// row_pos (device [state B], np = 1, t0 = 0): sequence b transitions at position row_pos[b] + 1;
// the RLT-2 register is then left to the caller.
// pos_max (row_pos only): the largest position any row of the pass reaches.
void decoder_pass(rlt_model* m, rlt_state* s, int t0, int np, hipStream_t st, const SliceBufs& sb,
                  const int* pos_dev = nullptr, const PassIO& io = PassIO(), const int* row_pos = nullptr,
                  int pos_max = 0) {
  const rlt_config& c = m->cfg;
  const Dt dt = m->dt;
  const int d = c.d, hd = m->hd, f = c.ffn, H = c.n_heads, dh = c.d_head, B = sb.B, Tm = s->Tm;
  const int rows = B * np;
  const RowMap zm = contiguous(d);
  const int A = m->act, ad = A * d, ahd = A * hd, af = A * f;
  const int64_t sd = A > 1 ? d : 0, shd = A > 1 ? hd : 0, sf = A > 1 ? f : 0;
  const int* rp = row_pos ? row_pos + sb.b0 : nullptr;
  // Folded RMSNorm on the 16-bit decode GEMMs: each residual GEMM also writes act(z * gain of
  // the next norm) and per-16-feature sums of squares; the next GEMM scales its rows by the
  // inverse RMS. The merge folds the first block's norm the same way (8-feature partials) when
  // the pass has one position; otherwise the first norm of the pass comes from the norm kernel.
  const bool fold = !m->batch_invariant && dt != Dt::F32 && rows <= kSkinnyMaxRows && d / 16 <= 256;
  const bool chain = fold && c.variant == RLT_V1 && c.L_D > 0;
  const bool merge_fold = fold && c.variant != RLT_V0 && c.L_D > 0 && np == 1 && d / 8 <= 256;
  if (c.variant == RLT_V0) {
    RowMap em; em.tn = np; em.sb = (int64_t)Tm * d; em.st = d;
    if (rp) { em.pos = rp; em.pst = d; }
    copy_rows(sb.e + (int64_t)t0 * d, em, sb.z, zm, rows, d, st);
  } else {
    // merge (eq 2.9-2.11): r = RMSNorm_s(s_{t-1} or the RLT-2 register), gate and state projection
    EpArgs a;
    if (chain && io.in_folded) {
      a.rs_ssp = sb.sssp; a.rs_n = d / 16; a.rs_d = d; a.rs_eps = c.rms_eps;
    } else {
      const float* src = c.variant == RLT_V1 ? sb.s : sb.rho;
      rmsnorm(dt, src, contiguous(d), m->ns, sb.xs, ad, B, d, c.rms_eps, st, sd);
    }
    a.resid = sb.z; a.rmap = zm; a.e = sb.e + (int64_t)t0 * d; a.gpre = sb.gpre + (int64_t)t0 * d;
    a.eb = (int64_t)Tm * d; a.et = d; a.nrep = np; a.alpha = c.alpha; a.x_split = A > 1;
    if (pos_dev) { a.e = sb.e; a.gpre = sb.gpre; a.pos_dev = pos_dev; a.pos_stride = d; }
    if (rp) { a.e = sb.e; a.gpre = sb.gpre; a.row_pos = rp; a.pos_stride = d; }
    if (merge_fold) {
      a.fold_zb = sb.xa; a.fold_ld = ad; a.out_split = sd; a.fold_ssp = sb.dssp; a.fold_gain = m->dec[0].n1;
    }
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::Merge, a, sb.xs, ad, m->wsr, B, 2 * d, d, st);
  }
  const float scale = 1.f / std::sqrt((float)dh);
  auto norm_in = [&](EpArgs& a, const float* gain) {
    if (fold) {
      a.rs_ssp = sb.dssp; a.rs_n = d / 16; a.rs_d = d; a.rs_eps = c.rms_eps;
    } else {
      rmsnorm(dt, sb.z, zm, gain, sb.xa, ad, rows, d, c.rms_eps, st, sd);
    }
  };
  auto fold_out = [&](EpArgs& r, const float* gain_next) {
    if (fold && gain_next) {
      r.fold_zb = sb.xa; r.fold_ld = ad; r.out_split = sd; r.fold_ssp = sb.dssp; r.fold_gain = gain_next;
    }
  };
  if (fold && c.L_D > 0 && !merge_fold)
    rmsnorm(dt, sb.z, zm, m->dec[0].n1, sb.xa, ad, rows, d, c.rms_eps, st, sd);
  for (int l = 0; l < c.L_D; ++l) {
    const LayerW& L = m->dec[l];
    // causal sliding-window self-attention over the ring (current key written first)
    EpArgs a;
    if (l > 0 || !fold) norm_in(a, L.n1);
    else if (merge_fold) { a.rs_ssp = sb.dssp; a.rs_n = d / 8; a.rs_d = d; a.rs_eps = c.rms_eps; }
    a.out = sb.q; a.ldo = hd; a.rope = s->rope; a.H = H; a.dh = dh; a.hd = hd; a.tn = np; a.pos0 = t0;
    a.x_split = A > 1; a.pos_dev = pos_dev; a.row_pos = rp;
    const int64_t ro = (int64_t)l * s->B * H * s->R * dh * m->esz;   // layer stride spans every sequence
    a.kv.k = (char*)sb.ring_k + ro; a.kv.v = (char*)sb.ring_v + ro; a.kv.cap = s->R; a.kv.ring = 1;
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::QKV, a, sb.xa, ad, L.wqkv, rows, 3 * hd, d, st);
    AttnArgs at;
    at.wide = !m->batch_invariant;
    at.q = sb.q; at.ldq = hd; at.k = a.kv.k; at.v = a.kv.v; at.kv_bstride = (int64_t)H * s->R * dh;
    at.cap = s->R; at.ring = 1; at.out = sb.ao; at.ldo = ahd; at.out_split = shd;
    at.B = B; at.nq = np; at.H = H; at.dh = dh;
    at.pos0 = t0; at.window = c.window; at.scale = scale; at.pos_dev = pos_dev; at.row_pos = rp;
    const int pmax = pos_dev ? 0 : (rp ? pos_max : t0 + np);
    attn_split(m, s, at, sb.slice, std::min(pmax, c.window));
    // passes of many positions (RLT-0) attend on MFMA tiles that the pass's queries of a
    // (sequence, head) share: the window and prefix masks of the flash kernel
    const bool tiles = np >= 16 && !m->batch_invariant && !pos_dev && !rp;
    // launches that read more keys and values than the last-level cache holds stream them with
    // the nontemporal hint (bytes of the longest range, every row)
    const int64_t kv_row = 2 * (int64_t)hd * m->esz;
    at.stream = (int64_t)B * std::min(pmax > 0 ? pmax : s->cap, c.window) * kv_row > kStreamBytes;
    timed(m, RLT_TIME_WINDOW_ATTN, st, [&] {
      if (!(tiles && attn_prefill(dt, at, st))) attn_decode(dt, at, st);
    });
    EpArgs r; r.resid = sb.z; r.rmap = zm; r.x_split = A > 1;
    fold_out(r, L.n2);
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::Residual, r, sb.ao, ahd, L.wo, rows, d, hd, st);
    // cross-attention to the prefix memory M_<=t of this layer's group
    EpArgs qx;
    norm_in(qx, L.n2);
    qx.out = sb.q; qx.ldo = hd; qx.rope = s->rope; qx.dh = dh; qx.tn = np; qx.pos0 = t0; qx.x_split = A > 1;
    qx.pos_dev = pos_dev; qx.row_pos = rp;
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::RopeQ, qx, sb.xa, ad, L.xq, rows, hd, d, st);
    const int g = c.groups == 1 ? 0 : l;
    const int64_t go = (int64_t)g * s->B * H * Tm * dh * m->esz;
    at.k = (char*)sb.mem_k + go; at.v = (char*)sb.mem_v + go; at.kv_bstride = (int64_t)H * Tm * dh;
    at.cap = Tm; at.ring = 0; at.window = 0;
    at.split_ws = nullptr;
    attn_split(m, s, at, sb.slice, pmax);
    at.memory = 1;
    at.stream = (int64_t)B * (pmax > 0 ? pmax : s->cap) * kv_row > kStreamBytes;
    timed(m, RLT_TIME_MEMORY_ATTN, st, [&] {
      if (!(tiles && attn_prefill(dt, at, st))) attn_decode(dt, at, st);
    });
    EpArgs r2; r2.resid = sb.z; r2.rmap = zm; r2.x_split = A > 1;
    fold_out(r2, L.n3);
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::Residual, r2, sb.ao, ahd, L.xo, rows, d, hd, st);
    // SwiGLU FFN
    EpArgs sw;
    norm_in(sw, L.n3);
    sw.out = sb.hid; sw.ldo = af; sw.out_split = sf; sw.x_split = A > 1;
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::SwiGLU, sw, sb.xa, ad, L.w13, rows, 2 * f, d, st);
    EpArgs r3; r3.resid = sb.z; r3.rmap = zm; r3.x_split = A > 1;
    fold_out(r3, l + 1 < c.L_D ? m->dec[l + 1].n1 : nullptr);
    if (l + 1 == c.L_D) {
      // the pass's outputs: s_t (last position of each sequence), the readout rows, and the
      // next merge's folded input
      r3.tn = np; r3.dup_last = sb.s; r3.dup_last_ld = d;
      r3.dup_rows = io.rows; r3.dup_map = io.rows_map;
      if (chain && io.out_fold) {
        r3.fold_zb = sb.xs; r3.fold_ld = ad; r3.out_split = sd; r3.fold_ssp = sb.sssp; r3.fold_gain = m->ns;
      }
    }
    mgemm(m, s, sb.slice, RLT_TIME_DECODER_GEMM, dt, Ep::Residual, r3, sb.hid, af, L.w2, rows, d, f, st);
  }
  if (c.L_D == 0) {
    // s_t = the last position's output of every sequence
    RowMap last; last.tn = 1; last.sb = (int64_t)np * d;
    copy_rows(sb.z + (int64_t)(np - 1) * d, last, sb.s, zm, B, d, st);
    if (io.rows) copy_rows(sb.z, zm, io.rows, io.rows_map, rows, d, st);
  }
  if (c.variant == RLT_V2 && !rp && (t0 + np) % c.chunk == 0)
    HIPCHK(hipMemcpyAsync(sb.rho, sb.s, sizeof(float) * B * d, hipMemcpyDeviceToDevice, st));
}

struct ScanOut {
  float* logits = nullptr;          // rows (b, c) at logits + (b * ld_b + c) * V
  int64_t ld_b = 0;
  float* s_out = nullptr;           // rows (b, c) at s_out + (b * ld_b + c) * d
  const int32_t* tok = nullptr;     // next token of (b, c) at tok[b * tok_ld + c]
  int64_t tok_ld = 0;
  float* lp = nullptr;              // log-prob of (b, c) at lp[b * lp_ld + c]
  int64_t lp_ld = 0;
  int lp_valid = 1 << 30;           // columns c >= lp_valid are not written
};

// Readout of buffered positions c0 .. c0+n-1 (scan-relative) of sequences b0 .. b0+nb-1, held in
// sbuf [B][kReadoutPositions][d] (or at src with sequence stride src_sb).
void readout(rlt_model* m, rlt_state* s, int c0, int n, const ScanOut& o, hipStream_t st, int b0, int nb,
             const float* src = nullptr, int64_t src_sb = 0, int slice = 0) {
  const rlt_config& c = m->cfg;
  const Dt dt = m->dt;
  const int d = c.d, V = c.vocab;
  const int rows = nb * n;
  RowMap sm; sm.tn = n; sm.sb = src ? src_sb : (int64_t)kReadoutPositions * d; sm.st = d;
  if (!src) src = s->sbuf + (int64_t)b0 * kReadoutPositions * d;
  const int A = m->act;
  void* xr = (char*)s->xr + (int64_t)b0 * kReadoutPositions * A * d * m->esz;
  float* lbuf = s->lbuf + (int64_t)b0 * kReadoutPositions * V;
  if (o.s_out) {
    RowMap dm; dm.tn = n; dm.sb = o.ld_b * d; dm.st = d;
    copy_rows(src, sm, o.s_out + ((int64_t)b0 * o.ld_b + c0) * d, dm, rows, d, st);
  }
  if (!o.logits && !o.lp) return;
  rmsnorm(dt, src, sm, m->nO, xr, A * d, rows, d, c.rms_eps, st, A > 1 ? d : 0);
  EpArgs a; a.out = lbuf; a.ldo = V; a.x_split = A > 1;
  mgemm(m, s, slice, RLT_TIME_DECODER_GEMM, dt, Ep::StoreF32, a, xr, A * d, m->wout, rows, V, d, st);
  if (o.logits) {
    RowMap dm; dm.tn = n; dm.sb = o.ld_b * V; dm.st = V;
    copy_rows(lbuf, contiguous(V), o.logits + ((int64_t)b0 * o.ld_b + c0) * V, dm, rows, V, st);
  }
  if (o.lp) {
    const int nv = std::min(n, o.lp_valid - c0);
    if (nv > 0) {
      RowMap lm; lm.tn = nv; lm.sb = (int64_t)n * V; lm.st = V;
      RowMap tm; tm.tn = nv; tm.sb = o.tok_ld; tm.st = 1;
      RowMap om; om.tn = nv; om.sb = o.lp_ld; om.st = 1;
      logprob(lbuf, lm, o.tok + (int64_t)b0 * o.tok_ld + c0, tm, o.lp + (int64_t)b0 * o.lp_ld + c0, om, nb * nv,
              V, st);
    }
  }
}

// Work split of the persistent scan: 1 group of every block (grid-wide barriers), or
// 8 * k groups (k blocks per CU, each group on one XCD owning batch / (8k) sequences).
// Groups pay for streaming the step's decoder weights once per group (from the 256 MB
// last-level cache), so they are chosen only when those weights are small.
int scan_groups(rlt_model* m, rlt_state* s) {
  const int B = s->B;
  switch (m->scan_mode) {
    case 3: return 1;
    case 4: return B % 8 == 0 ? 8 : 1;
    case 5: return B % 16 == 0 ? 16 : (B % 8 == 0 ? 8 : 1);
    case 6: return B % 32 == 0 ? 32 : (B % 16 == 0 ? 16 : (B % 8 == 0 ? 8 : 1));
    default: break;
  }
  const rlt_config& c = m->cfg;
  const int64_t w = (int64_t)c.L_D * (4 * (int64_t)m->hd * c.d + 2 * (int64_t)c.d * m->hd + 3 * (int64_t)c.d * c.ffn) +
                    2 * (int64_t)c.d * c.d;
  if (w * (int64_t)m->esz > (int64_t)96 << 20) return 1;
  if (B % 16 == 0) return 16;
  return B % 8 == 0 ? 8 : 1;
}

// Automatic mode runs one launch sequence per position: on MI355X at the algorithmic-task
// shape it measured faster than the persistent kernel, whose phases are bound by the
// latency of reading activations just written by other CUs.
bool use_persistent(rlt_model* m, rlt_state* s) {
  return s->scan_ok && m->scan_mode >= 2 && m->scan_mode <= 6 && !m->batch_invariant;
}

// Batch slices of the launch-path scan (each an independent chain on its own stream).
int scan_slices(rlt_model* m, rlt_state* s) {
  int want = 1;
  if (m->scan_mode == 7) want = 2;
  else if (m->scan_mode == 8) want = 4;
  return std::max(1, std::min(want, s->B));
}

void persistent_scan(rlt_model* m, rlt_state* s, int T, const ScanOut& o, hipStream_t st) {
  const rlt_config& c = m->cfg;
  const int d = c.d, start = s->n_dec;
  ScanParams p{};
  p.B = s->B; p.d = d; p.hd = m->hd; p.H = c.n_heads; p.dh = c.d_head; p.f = c.ffn; p.L = c.L_D;
  p.W = c.window; p.R = s->R; p.Tm = s->Tm; p.variant = (int)c.variant; p.chunk = c.chunk; p.P = s->P;
  p.ngroups = scan_groups(m, s);
  p.cpx = scan_cus() / 8;
  p.alpha = c.alpha; p.eps = c.rms_eps; p.scale = 1.f / std::sqrt((float)c.d_head);
  p.wsr = (const bf16_t*)m->wsr; p.ns = m->ns;
  p.g_first = c.L_D > 0 ? m->dec[0].n1 : m->ns;
  p.e = s->e; p.gpre = s->gpre; p.s = s->s; p.rho = s->rho;
  p.rhob = (bf16_t*)s->rhob; p.rhoss = s->rhoss; p.rope = s->rope;
  for (int i = 0; i < 2; ++i) { p.z[i] = s->pz[i]; p.zb[i] = (bf16_t*)s->pzb[i]; p.ssp[i] = s->pssp[i]; }
  p.q = (bf16_t*)s->pq; p.ao = (bf16_t*)s->pao; p.hid = (bf16_t*)s->phid;
  p.sall = s->sall; p.start = start; p.T = T; p.bar = s->bar; p.layer = s->layers_dev;
  fill_zero_u32(s->bar, kBarWords, st);
  int grid = 0;
  hipError_t e = launch_scan(p, &grid, st);
  if (e != hipSuccess) fail(RLT_ERR_HIP, std::string("persistent scan launch: ") + hipGetErrorString(e));
  s->scan_grid = grid;
  HIPCHK(hipMemcpyAsync(s->abort_host, s->bar + 64 * 10, sizeof(int), hipMemcpyDeviceToHost, st));
  s->block_steps += (int64_t)c.L_D * (c.variant == RLT_V1 ? T
                                       : c.variant == RLT_V2 ? ((start + T - 1) / c.chunk - start / c.chunk + 1)
                                                             : (T + s->P - 1) / s->P);
  s->n_dec = start + T;
  if (o.logits || o.lp || o.s_out) {
    for (int c0 = 0; c0 < T; c0 += kReadoutPositions) {
      const int n = std::min(kReadoutPositions, T - c0);
      readout(m, s, c0, n, o, st, 0, s->B, s->sall + (int64_t)(start + c0) * d, (int64_t)s->Tm * d);
    }
  }
  check_launch();
}

// One RLT-1 position of the launch path, captured once per state as a HIP graph and replayed
// for every position: the kernels read the position from s->pos_dev, advanced by the graph's
// last kernel. Replaying saves the per-launch submission cost (measured: 2.6 -> 1.7 us per
// dependent kernel). The readout stays eager every kReadoutPositions positions.
hipGraphExec_t pass_graph(rlt_model* m, rlt_state* s, bool want_rows, bool in_folded) {
  hipGraphExec_t& ge = s->pass_graph[want_rows ? 1 : 0][in_folded ? 1 : 0];
  if (ge) return ge;
  const int d = m->cfg.d;
  hipStream_t cs = s->sub[0];
  const SliceBufs sb = slice_bufs(m, s, 0, s->B);
  HIPCHK(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
  PassIO io;
  io.in_folded = in_folded;
  io.out_fold = true;
  decoder_pass(m, s, 0, 1, cs, sb, s->pos_dev, io);
  if (want_rows) {
    RowMap dm; dm.tn = 1; dm.sb = (int64_t)kReadoutPositions * d; dm.st = d;
    copy_rows_at(sb.z, contiguous(d), s->sbuf, dm, s->pos_dev + 1, d, s->B, d, cs);
  }
  advance_scan_pos(s->pos_dev, 1, cs);
  hipGraph_t g = nullptr;
  const hipError_t e1 = hipGetLastError();
  const hipError_t e2 = hipStreamEndCapture(cs, &g);
  if (e1 != hipSuccess || e2 != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    fail(RLT_ERR_HIP, std::string("scan graph capture: ") + hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  }
  const hipError_t e3 = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e3 != hipSuccess) {
    ge = nullptr;
    fail(RLT_ERR_HIP, std::string("scan graph instantiate: ") + hipGetErrorString(e3));
  }
  return ge;
}

// Explicit only: measured at the algorithmic shape the replayed graph (44.2 ms per 64x257 scan)
// is not faster than the stream-ordered launches (43.2 ms), whose dispatch already overlaps.
bool use_graph(rlt_model* m, rlt_state* s) {
  return m->cfg.variant == RLT_V1 && m->cfg.L_D > 0 && scan_slices(m, s) == 1 && m->scan_mode == 9 &&
         !m->batch_invariant;
}

void graph_scan(rlt_model* m, rlt_state* s, int T, const ScanOut& o, hipStream_t st) {
  const int start = s->n_dec;
  const bool want_rows = o.logits || o.lp || o.s_out;
  // the first replay of the call normalizes s_{t-1} itself; later replays take the folded
  // merge input the previous replay wrote (the launch path's chaining)
  hipGraphExec_t ge0 = pass_graph(m, s, want_rows, false), ge1 = pass_graph(m, s, want_rows, true);
  set_scan_pos(s->pos_dev, start, 0, st);
  int c0 = 0, buffered = 0;
  for (int done = 0; done < T; ++done) {
    if (want_rows && buffered == kReadoutPositions) {
      readout(m, s, c0, buffered, o, st, 0, s->B);
      c0 += buffered;
      buffered = 0;
      set_scan_pos(s->pos_dev, start + done, 0, st);
    }
    HIPCHK(hipGraphLaunch(done == 0 ? ge0 : ge1, st));
    s->block_steps += m->cfg.L_D;
    if (want_rows) buffered += 1;
    s->n_dec = start + done + 1;
  }
  if (want_rows && buffered > 0) readout(m, s, c0, buffered, o, st, 0, s->B);
  check_launch();
}

void do_scan(rlt_model* m, rlt_state* s, int T, const ScanOut& o, hipStream_t st) {
  if (use_persistent(m, s)) {
    persistent_scan(m, s, T, o, st);
    return;
  }
  if (use_graph(m, s)) {
    graph_scan(m, s, T, o, st);
    return;
  }
  const rlt_config& c = m->cfg;
  const int d = c.d;
  const int start = s->n_dec;
  const bool want_rows = o.logits || o.lp || o.s_out;
  // batch slices: independent chains of sequences, each on its own stream
  const int ns = scan_slices(m, s);
  std::vector<SliceBufs> sl(ns);
  std::vector<hipStream_t> ss(ns, st);
  for (int k = 0; k < ns; ++k) {
    const int b0 = (int)((int64_t)s->B * k / ns), b1 = (int)((int64_t)s->B * (k + 1) / ns);
    sl[k] = slice_bufs(m, s, b0, b1 - b0);
    sl[k].slice = k;
    if (ns > 1) ss[k] = s->sub[k];
  }
  if (ns > 1) {
    HIPCHK(hipEventRecord(s->ev_fork, st));
    for (int k = 0; k < ns; ++k) HIPCHK(hipStreamWaitEvent(ss[k], s->ev_fork, 0));
  }
  int c0 = 0;          // scan-relative column of the first buffered position
  int buffered = 0;
  int done = 0;
  auto flush = [&] {
    if (buffered > 0)
      for (int k = 0; k < ns; ++k) readout(m, s, c0, buffered, o, ss[k], sl[k].b0, sl[k].B, nullptr, 0, k);
    c0 += buffered;
    buffered = 0;
  };
  while (done < T) {
    const int t0 = start + done;
    int np = 1;
    if (c.variant == RLT_V2) np = std::min(T - done, (t0 / c.chunk + 1) * c.chunk - t0);
    else if (c.variant == RLT_V0) np = std::min(T - done, s->P);
    if (want_rows && buffered + np > kReadoutPositions) flush();
    for (int k = 0; k < ns; ++k) {
      PassIO io;
      io.in_folded = done > 0;
      io.out_fold = done + np < T;
      if (want_rows) {
        io.rows = s->sbuf + ((int64_t)sl[k].b0 * kReadoutPositions + buffered) * d;
        io.rows_map.tn = np; io.rows_map.sb = (int64_t)kReadoutPositions * d; io.rows_map.st = d;
      }
      decoder_pass(m, s, t0, np, ss[k], sl[k], nullptr, io);
    }
    s->block_steps += c.L_D;
    if (want_rows) buffered += np;
    done += np;
    s->n_dec = t0 + np;
  }
  if (want_rows) flush();
  if (ns > 1) {
    for (int k = 0; k < ns; ++k) {
      HIPCHK(hipEventRecord(s->ev_join[k], ss[k]));
      HIPCHK(hipStreamWaitEvent(st, s->ev_join[k], 0));
    }
  }
  check_launch();
}

// ------------------------------------------------------------------ rows at their own positions
// Batch-wide calls need every row at one position (and the state leaves the per-row mode then).
void leave_ragged(rlt_state* s) {
  if (!s->ragged) return;
  for (int b = 1; b < s->B; ++b)
    if (s->row_n[b] != s->row_n[0])
      fail(RLT_ERR_ORDER, "rows are at different positions: use rlt_step_rows / rlt_state_reset_rows, or "
                          "reset the state");
  s->n_enc = s->n_dec = s->row_n[0];
  s->ragged = false;
}

void enter_ragged(rlt_state* s) {
  if (s->ragged) return;
  if (s->n_dec != s->n_enc) fail(RLT_ERR_ORDER, "consume the encoded positions before per-row calls");
  s->row_n.assign(s->B, s->n_dec);
  s->ragged = true;
}

// Copies v (3 arrays of B ints) to rp_dev on the stream through a pinned slot; a slot is
// rewritten only after the copy that last read it has run.
void stage_rows(rlt_state* s, const std::vector<int>& v, hipStream_t st) {
  const int k = s->rp_next;
  s->rp_next = (k + 1) % kStage;
  if (s->rp_used[k]) HIPCHK(hipEventSynchronize(s->rp_ev[k]));
  int* h = s->rp_host + (size_t)k * 3 * s->B;
  std::memcpy(h, v.data(), sizeof(int) * 3 * s->B);
  HIPCHK(hipMemcpyAsync(s->rp_dev, h, sizeof(int) * 3 * s->B, hipMemcpyHostToDevice, st));
  HIPCHK(hipEventRecord(s->rp_ev[k], st));
  s->rp_used[k] = true;
}

// One position for every row with active[b] != 0, each at its own position row_n[b] + 1: the
// encoder step, memory append and transition of generation F.2 (summary appendix F.2), batched
// over rows at unequal positions. Rows that do not move run the same kernels at position
// row_n[b] + 1 (keys, memory and encoder rows land beyond their prefix, in the slack position
// when the row is full, or in the ring slot of a position the window has already left) and
// get their s back afterwards, so their state is unchanged.
void step_rows(rlt_model* m, rlt_state* s, const int32_t* tokens, const int32_t* active, float* logits,
               hipStream_t st) {
  const rlt_config& c = m->cfg;
  const int B = s->B, d = c.d;
  std::vector<int> v(3 * B, 0);
  int moving = 0;
  for (int b = 0; b < B; ++b) {
    const bool a = active[b] != 0;
    v[b] = s->row_n[b];
    v[B + b] = a ? 0 : 1;
    v[2 * B + b] = (a && c.variant == RLT_V2 && (s->row_n[b] + 1) % c.chunk == 0) ? 1 : 0;
    moving += a ? 1 : 0;
  }
  if (!moving) return;
  stage_rows(s, v, st);
  const int* pos = s->rp_dev;
  const int* keep = s->rp_dev + B;
  const int* reg = s->rp_dev + 2 * B;
  active_tokens(tokens, keep, s->rtok, B, st);
  HIPCHK(hipMemcpyAsync(s->s_bak, s->s, sizeof(float) * B * d, hipMemcpyDeviceToDevice, st));
  const int pmax = *std::max_element(s->row_n.begin(), s->row_n.end()) + 1;
  do_encode(m, s, s->rtok, 1, st, pos, pmax);
  const SliceBufs sb = slice_bufs(m, s, 0, B);
  PassIO io;
  io.rows = s->sbuf;
  io.rows_map.tn = 1; io.rows_map.sb = (int64_t)kReadoutPositions * d; io.rows_map.st = d;
  decoder_pass(m, s, 0, 1, st, sb, nullptr, io, pos, pmax);
  ScanOut o;
  o.logits = logits; o.ld_b = 1;
  readout(m, s, 0, 1, o, st, 0, B);
  if (c.variant == RLT_V2) masked_rows(s->s, d, s->rho, reg, B, d, st);
  masked_rows(s->s_bak, d, s->s, keep, B, d, st);
  check_launch();
  s->block_steps += c.L_D;
  for (int b = 0; b < B; ++b)
    if (active[b]) s->row_n[b] += 1;
}

// ------------------------------------------------------------------ snapshots
// Payload of a prefix snapshot, in this order (B sequences, n_enc encoded and n_dec consumed
// positions; every part contiguous):
//   s, rho            fp32 [B][d] each
//   rings C^D k, v    [L_D][B][H][R][dh] each (whole rings: slots are (position - 1) mod R)
//   memory M k, v     [G][B][H][n_enc][dh] each (the encoded prefix of every group)
//   encoder C^E k, v  [L_E][B][H][n_enc][dh] each, when the state keeps the encoder cache
//   e, gpre           fp32 [B][n_enc - n_dec][d] (encoded, not yet consumed positions)
// Element width esz for the caches, memory and rings.
struct SnapPart {
  char* state;        // first byte in the state (row 0)
  int64_t rows;       // rows of the part
  int64_t width;      // bytes copied per row
  int64_t pitch;      // state row pitch in bytes
};
std::vector<SnapPart> snapshot_parts(rlt_model* m, rlt_state* s, int n_enc, int n_dec, bool with_enc) {
  const rlt_config& c = m->cfg;
  const int64_t B = s->B, d = c.d, H = c.n_heads, dh = c.d_head, e = m->esz, Tm = s->Tm;
  std::vector<SnapPart> v;
  v.push_back({(char*)s->s, 1, B * d * 4, B * d * 4});
  v.push_back({(char*)s->rho, 1, B * d * 4, B * d * 4});
  if (c.L_D > 0) {
    const int64_t rb = (int64_t)c.L_D * B * H * s->R * dh * e;
    v.push_back({(char*)s->ring_k, 1, rb, rb});
    v.push_back({(char*)s->ring_v, 1, rb, rb});
    const int64_t mr = (int64_t)c.groups * B * H;
    v.push_back({(char*)s->mem_k, mr, (int64_t)n_enc * dh * e, Tm * dh * e});
    v.push_back({(char*)s->mem_v, mr, (int64_t)n_enc * dh * e, Tm * dh * e});
  }
  if (with_enc) {
    const int64_t er = (int64_t)c.L_E * B * H;
    v.push_back({(char*)s->enc_k, er, (int64_t)n_enc * dh * e, Tm * dh * e});
    v.push_back({(char*)s->enc_v, er, (int64_t)n_enc * dh * e, Tm * dh * e});
    if (s->enc_lo > 0) {   // lo planes of two-term keys and values
      v.push_back({(char*)s->enc_k + s->enc_lo * e, er, (int64_t)n_enc * dh * e, Tm * dh * e});
      v.push_back({(char*)s->enc_v + s->enc_lo * e, er, (int64_t)n_enc * dh * e, Tm * dh * e});
    }
  }
  const int64_t pend = (int64_t)(n_enc - n_dec) * d * 4;
  v.push_back({(char*)(s->e + (int64_t)n_dec * d), B, pend, Tm * d * 4});
  if (s->gpre) v.push_back({(char*)(s->gpre + (int64_t)n_dec * d), B, pend, Tm * d * 4});
  return v;
}

int64_t snapshot_payload(const std::vector<SnapPart>& parts) {
  int64_t n = 0;
  for (const SnapPart& p : parts) n += p.rows * p.width;
  return n;
}

// to_state = false: state -> buf; true: buf -> state. buf may be device or host memory.
void snapshot_copy(const std::vector<SnapPart>& parts, char* buf, bool to_state, hipStream_t st) {
  int64_t off = 0;
  for (const SnapPart& p : parts) {
    if (p.rows > 0 && p.width > 0) {
      if (to_state)
        HIPCHK(hipMemcpy2DAsync(p.state, p.pitch, buf + off, p.width, p.width, p.rows, hipMemcpyDefault, st));
      else
        HIPCHK(hipMemcpy2DAsync(buf + off, p.width, p.state, p.pitch, p.width, p.rows, hipMemcpyDefault, st));
    }
    off += p.rows * p.width;
  }
}

}  // namespace

// ======================================================================= C ABI
extern "C" {

const char* rlt_status_string(int status) {
  switch (status) {
    case RLT_OK: return "ok";
    case RLT_ERR_INVALID_ARG: return "invalid argument";
    case RLT_ERR_UNSUPPORTED: return "unsupported";
    case RLT_ERR_OOM: return "out of device memory";
    case RLT_ERR_CAPACITY: return "capacity exceeded";
    case RLT_ERR_STALE_STATE: return "stale state";
    case RLT_ERR_HIP: return "HIP error";
    case RLT_ERR_ORDER: return "decoder ahead of encoder";
    default: return "unknown status";
  }
}

const char* rlt_last_error(void) { return g_err.c_str(); }

int rlt_create(const rlt_config* cfg, const rlt_tensor* weights, int n_weights, hipStream_t stream, rlt_model** out) {
  return guarded([&] {
    if (!cfg || !out) fail(RLT_ERR_INVALID_ARG, "null config or output");
    *out = nullptr;
    validate_config(*cfg);
    auto W = index_weights(*cfg, weights, n_weights);
    auto* m = new rlt_model();
    try {
      m->cfg = *cfg;
      HIPCHK(hipGetDevice(&m->device));
      m->dt = cfg->dtype == RLT_FP32 ? Dt::F32 : (cfg->dtype == RLT_BF16 ? Dt::BF16 : Dt::F16);
      m->act = cfg->dtype == RLT_FP16X2 ? 2 : 1;
      m->esz = cfg->dtype == RLT_FP32 ? 4 : 2;
      m->hd = cfg->n_heads * cfg->d_head;
      // RLT_SKINNY_TILE=<TPW>x<NMB>[x<S>]: every decode GEMM of this model whose shape admits it
      // takes that tile shape and K split count instead of the cost model's (tile measurements)
      if (const char* env = getenv("RLT_SKINNY_TILE")) {
        int t = 0, n = 0, z = 1;
        if (sscanf(env, "%dx%dx%d", &t, &n, &z) >= 2) {
          m->tile_ov[0] = t;
          m->tile_ov[1] = n;
          m->tile_ov[2] = z;
        }
      }
      size_t total = 0;
      layout_model(m, nullptr, &total);
      if (hipMalloc(&m->arena, total) != hipSuccess) fail(RLT_ERR_OOM, "weight arena allocation failed");
      m->arena_bytes = total;
      layout_model(m, (char*)m->arena, &total);
      fill_zero_u32(m->arena, (int64_t)(total / 4), stream);   // padding rows of tile-major weights
      pack_all(m, W, stream);
      HIPCHK(hipStreamSynchronize(stream));
      m->wdigest = weights_digest(m, stream);
    } catch (...) {
      if (m->arena) (void)hipFree(m->arena);
      delete m;
      throw;
    }
    *out = m;
  });
}

int rlt_update_weights(rlt_model* m, const rlt_tensor* weights, int n_weights, hipStream_t stream) {
  return guarded([&] {
    if (!m) fail(RLT_ERR_INVALID_ARG, "null model");
    auto W = index_weights(m->cfg, weights, n_weights);
    pack_all(m, W, stream);
    HIPCHK(hipStreamSynchronize(stream));
    m->wdigest = weights_digest(m, stream);
    m->version += 1;
  });
}

int rlt_destroy(rlt_model* m) {
  return guarded([&] {
    if (!m) fail(RLT_ERR_INVALID_ARG, "null model");
    if (m->n_states > 0) fail(RLT_ERR_INVALID_ARG, "destroy the model's states first");
    if (m->arena) HIPCHK(hipFree(m->arena));
    for (auto& list : m->timed)
      for (auto& pr : list) {
        HIPCHK(hipEventDestroy(pr.first));
        HIPCHK(hipEventDestroy(pr.second));
      }
    for (hipEvent_t e : m->ev_free) HIPCHK(hipEventDestroy(e));
    delete m;
  });
}

int rlt_kernel_timing(rlt_model* m, int on) {
  return guarded([&] {
    if (!m) fail(RLT_ERR_INVALID_ARG, "null model");
    m->timing = on != 0;
  });
}

int rlt_kernel_time(rlt_model* m, int kind, double* total_ms, int64_t* launches) {
  return guarded([&] {
    if (!m || !total_ms || !launches) fail(RLT_ERR_INVALID_ARG, "null model or output");
    if (kind < 0 || kind >= RLT_TIME_KINDS) fail(RLT_ERR_INVALID_ARG, "unknown kernel kind");
    double tot = 0.0;
    auto& list = m->timed[kind];
    for (auto& pr : list) {
      HIPCHK(hipEventSynchronize(pr.second));
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, pr.first, pr.second));
      tot += ms;
      m->ev_free.push_back(pr.first);
      m->ev_free.push_back(pr.second);
    }
    *total_ms = tot;
    *launches = (int64_t)list.size();
    list.clear();
  });
}

int rlt_state_create(rlt_model* m, int batch, int max_len, int keep_encoder_cache, hipStream_t stream,
                     rlt_state** out) {
  return guarded([&] {
    if (!m || !out) fail(RLT_ERR_INVALID_ARG, "null model or output");
    *out = nullptr;
    if (batch < 1 || max_len < 1) fail(RLT_ERR_INVALID_ARG, "batch and max_len must be >= 1");
    if (max_len > 16384) fail(RLT_ERR_UNSUPPORTED, "max_len > 16384");
    const rlt_config& c = m->cfg;
    auto* s = new rlt_state();
    try {
      s->m = m;
      s->B = batch;
      s->Tm = max_len + 1;   // one slack position per sequence: a per-row step of a row that does not
                             // move writes its discarded keys, memory and encoder rows there when the
                             // row is full
      s->cap = max_len;
      s->keep_enc = keep_encoder_cache ? 1 : 0;
      s->P = c.variant == RLT_V2 ? c.chunk : (c.variant == RLT_V0 ? std::min(kParallelPositions, max_len) : 1);
      s->R = c.window + s->P - 1;
      const int64_t B = batch, Tm = s->Tm, d = c.d, hd = m->hd, f = c.ffn, V = c.vocab, H = c.n_heads,
                    dh = c.d_head;
      const size_t e = m->esz;
      // two-term encoder attention operands (with two-term GEMM inputs): C^E holds a lo plane
      const int64_t EA = m->act;
      if (s->keep_enc) {
        const int64_t plane = (int64_t)c.L_E * B * H * Tm * dh;
        s->enc_k = dev_alloc(s, (size_t)(EA * plane) * e, 0, EA * c.L_E * B * H * max_len * dh * (int64_t)e);
        s->enc_v = dev_alloc(s, (size_t)(EA * plane) * e, 0, EA * c.L_E * B * H * max_len * dh * (int64_t)e);
        s->enc_lo = EA > 1 ? plane : 0;
      }
      if (c.L_D > 0) {
        s->mem_k = dev_alloc(s, (size_t)c.groups * B * H * Tm * dh * e, 1, (int64_t)c.groups * B * H * max_len * dh * e);
        s->mem_v = dev_alloc(s, (size_t)c.groups * B * H * Tm * dh * e, 1, (int64_t)c.groups * B * H * max_len * dh * e);
        s->ring_k = dev_alloc(s, (size_t)c.L_D * B * H * s->R * dh * e, 2);
        s->ring_v = dev_alloc(s, (size_t)c.L_D * B * H * s->R * dh * e, 2);
      }
      s->s = (float*)dev_alloc(s, sizeof(float) * B * d, 3);
      s->rho = (float*)dev_alloc(s, sizeof(float) * B * d, 3);
      s->e = (float*)dev_alloc(s, sizeof(float) * B * Tm * d, 4, (int64_t)sizeof(float) * B * max_len * d);
      if (c.variant != RLT_V0)
        s->gpre = (float*)dev_alloc(s, sizeof(float) * B * Tm * d, 4, (int64_t)sizeof(float) * B * max_len * d);
      s->rope = (float2*)dev_alloc(s, sizeof(float2) * (Tm + 1) * (dh / 2), 5);
      const int64_t rows = B * s->P;
      s->z = (float*)dev_alloc(s, sizeof(float) * rows * d, 5);
      const int64_t A = m->act;   // two-term activation rows are twice as wide
      s->xa = dev_alloc(s, rows * A * d * e, 5);
      s->dssp = (float*)dev_alloc(s, sizeof(float) * rows * (d / 8), 5);
      s->xs = dev_alloc(s, B * A * d * e, 5);
      s->sssp = (float*)dev_alloc(s, sizeof(float) * B * (d / 16), 5);
      s->q = dev_alloc(s, rows * hd * e, 5);
      s->ao = dev_alloc(s, rows * A * hd * e, 5);
      s->hid = dev_alloc(s, rows * A * f * e, 5);
      const int64_t rr = B * kReadoutPositions;
      s->sbuf = (float*)dev_alloc(s, sizeof(float) * rr * d, 5);
      s->xr = dev_alloc(s, rr * A * d * e, 5);
      s->lbuf = (float*)dev_alloc(s, sizeof(float) * rr * V, 5);
      s->enc_rows = std::min<int64_t>(B * Tm, std::max<int64_t>(kEncoderRows, Tm));
      const int64_t er = s->enc_rows;
      s->exa = dev_alloc(s, er * A * d * e, 5);
      s->eq = dev_alloc(s, er * A * hd * e, 5);
      s->eao = dev_alloc(s, er * A * hd * e, 5);
      s->ehid = dev_alloc(s, er * A * f * e, 5);
      if (!s->keep_enc) {
        s->ekv_k = dev_alloc(s, er * A * hd * e, 5);
        s->ekv_v = dev_alloc(s, er * A * hd * e, 5);
        s->ekv_lo = A > 1 ? er * hd : 0;
      }
      s->toks = (int32_t*)dev_alloc(s, sizeof(int32_t) * B * Tm, 5);
      s->glog = (float*)dev_alloc(s, sizeof(float) * B * V, 5);
      s->gtok = (int32_t*)dev_alloc(s, sizeof(int32_t) * B, 5);
      s->pos_dev = (int*)dev_alloc(s, 256, 5);
      s->lp = (float*)dev_alloc(s, sizeof(float) * B * Tm, 5);
      s->rp_dev = (int*)dev_alloc(s, sizeof(int) * 3 * B, 5);
      s->rtok = (int32_t*)dev_alloc(s, sizeof(int32_t) * B, 5);
      s->s_bak = (float*)dev_alloc(s, sizeof(float) * B * d, 5);
      s->attn_ws = (float*)dev_alloc(s, sizeof(float) * kMaxSlices * kAttnSplitBlocks * (dh + 2), 5);
      if (m->dt != Dt::F32) {
        // split-K workspace per slice: kMaxKSplit partial copies of the widest decode GEMM output
        // (rows of a decoder pass or an encoder step, at most 32 MB; wider launches run unsplit)
        const int64_t kr = (std::min<int64_t>(std::max<int64_t>(rows, B), kSkinnyMaxRows) + 63) / 64 * 64;
        const int64_t kn = (std::max({3 * hd, 2 * f, 2 * d}) + 63) / 64 * 64;
        s->kpart_slice = std::min<int64_t>((int64_t)kMaxKSplit * kr * kn, (int64_t)8 << 20);
        s->kpart = (float*)dev_alloc(s, sizeof(float) * kMaxSlices * s->kpart_slice, 5);
      }
      s->samp_ws = dev_alloc(s, (size_t)sample_workspace_bytes((int)B, (int)V), 5);
      HIPCHK(hipHostMalloc((void**)&s->rp_host, sizeof(int) * kStage * 3 * B, hipHostMallocDefault));
      for (int k = 0; k < kStage; ++k) HIPCHK(hipEventCreateWithFlags(&s->rp_ev[k], hipEventDisableTiming));
      if (m->dt == Dt::BF16 && scan_supported((int)dh, (int)rows, (int)d, (int)hd, (int)f, (int)Tm, c.L_D)) {
        s->scan_ok = true;
        for (int i = 0; i < 2; ++i) {
          s->pz[i] = (float*)dev_alloc(s, sizeof(float) * rows * d, 5);
          s->pzb[i] = dev_alloc(s, rows * d * e, 5);
          s->pssp[i] = (float*)dev_alloc(s, sizeof(float) * rows * (d / 8), 5);
        }
        s->pq = dev_alloc(s, rows * hd * e, 5);
        s->pao = dev_alloc(s, rows * hd * e, 5);
        s->phid = dev_alloc(s, rows * f * e, 5);
        s->rhob = dev_alloc(s, B * d * e, 3);
        s->rhoss = (float*)dev_alloc(s, sizeof(float) * B * (d / 16), 3);
        s->sall = (float*)dev_alloc(s, sizeof(float) * B * Tm * d, 4);
        s->bar = (unsigned*)dev_alloc(s, sizeof(unsigned) * kBarWords, 5);
        std::vector<ScanLayer> Ls(c.L_D);
        for (int l = 0; l < c.L_D; ++l) {
          const LayerW& L = m->dec[l];
          ScanLayer& y = Ls[l];
          y.wqkv = (const bf16_t*)L.wqkv; y.wo = (const bf16_t*)L.wo; y.xq = (const bf16_t*)L.xq;
          y.xo = (const bf16_t*)L.xo; y.w13 = (const bf16_t*)L.w13; y.w2 = (const bf16_t*)L.w2;
          y.g1 = L.n1; y.g2 = L.n2; y.g3 = L.n3;
          y.gnext = l + 1 < c.L_D ? m->dec[l + 1].n1 : (c.variant == RLT_V0 ? m->nO : m->ns);
          const int g = c.groups == 1 ? 0 : l;
          y.mk = (const bf16_t*)((char*)s->mem_k + (int64_t)g * B * H * Tm * dh * e);
          y.mv = (const bf16_t*)((char*)s->mem_v + (int64_t)g * B * H * Tm * dh * e);
          y.rk = (bf16_t*)((char*)s->ring_k + (int64_t)l * B * H * s->R * dh * e);
          y.rv = (bf16_t*)((char*)s->ring_v + (int64_t)l * B * H * s->R * dh * e);
        }
        if (c.L_D > 0) {
          s->layers_dev = (ScanLayer*)dev_alloc(s, sizeof(ScanLayer) * c.L_D, 5);
          HIPCHK(hipMemcpy(s->layers_dev, Ls.data(), sizeof(ScanLayer) * c.L_D, hipMemcpyHostToDevice));
        }
        HIPCHK(hipHostMalloc((void**)&s->abort_host, sizeof(int), hipHostMallocDefault));
        *s->abort_host = 0;
      }
      for (int k = 0; k < kMaxSlices; ++k) {
        HIPCHK(hipStreamCreateWithFlags(&s->sub[k], hipStreamNonBlocking));
        HIPCHK(hipEventCreateWithFlags(&s->ev_join[k], hipEventDisableTiming));
      }
      HIPCHK(hipEventCreateWithFlags(&s->ev_fork, hipEventDisableTiming));
      rope_table(s->rope, (int)Tm + 1, (int)dh, c.rope_base, stream);
      check_launch();
      m->n_states += 1;
      *out = s;
      if (rlt_state_reset(m, s, stream) != RLT_OK) fail(RLT_ERR_HIP, g_err);
      HIPCHK(hipStreamSynchronize(stream));
    } catch (...) {
      if (*out) { m->n_states -= 1; *out = nullptr; }
      for (void* p : s->allocs) (void)hipFree(p);
      for (int k = 0; k < kMaxSlices; ++k) {
        if (s->sub[k]) (void)hipStreamDestroy(s->sub[k]);
        if (s->ev_join[k]) (void)hipEventDestroy(s->ev_join[k]);
      }
      if (s->ev_fork) (void)hipEventDestroy(s->ev_fork);
      if (s->abort_host) (void)hipHostFree(s->abort_host);
      if (s->rp_host) (void)hipHostFree(s->rp_host);
      for (int k = 0; k < kStage; ++k)
        if (s->rp_ev[k]) (void)hipEventDestroy(s->rp_ev[k]);
      delete s;
      throw;
    }
  });
}

int rlt_state_reset(rlt_model* m, rlt_state* s, hipStream_t stream) {
  return guarded([&] {
    if (!m || !s || s->m != m) fail(RLT_ERR_INVALID_ARG, "null or foreign state");
    const rlt_config& c = m->cfg;
    if (c.variant != RLT_V0) {
      broadcast_row(m->s0, s->s, s->B, c.d, stream);
      broadcast_row(m->s0, s->rho, s->B, c.d, stream);
    } else {
      HIPCHK(hipMemsetAsync(s->s, 0, sizeof(float) * s->B * c.d, stream));
    }
    check_launch();
    s->n_enc = 0;
    s->n_dec = 0;
    s->block_steps = 0;
    s->version = m->version;
    s->ragged = false;
  });
}

int rlt_state_destroy(rlt_state* s) {
  return guarded([&] {
    if (!s) fail(RLT_ERR_INVALID_ARG, "null state");
    for (auto& gw : s->pass_graph)
      for (auto& ge : gw)
        if (ge) HIPCHK(hipGraphExecDestroy(ge));
    for (void* p : s->allocs) HIPCHK(hipFree(p));
    if (s->abort_host) HIPCHK(hipHostFree(s->abort_host));
    for (int k = 0; k < kMaxSlices; ++k) {
      if (s->sub[k]) HIPCHK(hipStreamDestroy(s->sub[k]));
      if (s->ev_join[k]) HIPCHK(hipEventDestroy(s->ev_join[k]));
    }
    if (s->ev_fork) HIPCHK(hipEventDestroy(s->ev_fork));
    if (s->rp_host) HIPCHK(hipHostFree(s->rp_host));
    for (int k = 0; k < kStage; ++k)
      if (s->rp_ev[k]) HIPCHK(hipEventDestroy(s->rp_ev[k]));
    s->m->n_states -= 1;
    delete s;
  });
}

int rlt_state_bytes(const rlt_state* s, int64_t out[6]) {
  return guarded([&] {
    if (!s || !out) fail(RLT_ERR_INVALID_ARG, "null state or output");
    for (int i = 0; i < 6; ++i) out[i] = s->bytes[i];
  });
}

int rlt_state_positions(const rlt_state* s, int* n_encoded, int* n_decoded) {
  return guarded([&] {
    if (!s) fail(RLT_ERR_INVALID_ARG, "null state");
    int ne = s->n_enc, nd = s->n_dec;
    if (s->ragged) {
      for (int b = 1; b < s->B; ++b)
        if (s->row_n[b] != s->row_n[0]) fail(RLT_ERR_ORDER, "rows are at different positions (rlt_state_row_positions)");
      ne = nd = s->row_n[0];
    }
    if (n_encoded) *n_encoded = ne;
    if (n_decoded) *n_decoded = nd;
  });
}

int rlt_state_row_positions(const rlt_state* s, int32_t* n) {
  return guarded([&] {
    if (!s || !n) fail(RLT_ERR_INVALID_ARG, "null pointer");
    for (int b = 0; b < s->B; ++b) n[b] = s->ragged ? s->row_n[b] : s->n_dec;
  });
}

int rlt_step_rows(rlt_model* m, rlt_state* s, const int32_t* tokens, const int32_t* active, float* logits,
                  hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    if (!tokens || !active || !logits) fail(RLT_ERR_INVALID_ARG, "tokens, active and logits required");
    if (!s->enc_k) fail(RLT_ERR_UNSUPPORTED, "per-row steps need keep_encoder_cache");
    enter_ragged(s);
    for (int b = 0; b < s->B; ++b)
      if (active[b] && s->row_n[b] + 1 > s->cap) fail(RLT_ERR_CAPACITY, "a moving row would exceed max_len");
    step_rows(m, s, tokens, active, logits, stream);
  });
}

int rlt_state_reset_rows(rlt_model* m, rlt_state* s, const int32_t* rows, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    if (!rows) fail(RLT_ERR_INVALID_ARG, "rows required");
    enter_ragged(s);
    const int B = s->B, d = m->cfg.d;
    std::vector<int> v(3 * B, 0);
    int any = 0;
    for (int b = 0; b < B; ++b) {
      v[B + b] = rows[b] ? 1 : 0;
      any += v[B + b];
    }
    if (!any) return;
    stage_rows(s, v, stream);
    if (m->cfg.variant != RLT_V0) {
      masked_rows(m->s0, 0, s->s, s->rp_dev + B, B, d, stream);
      masked_rows(m->s0, 0, s->rho, s->rp_dev + B, B, d, stream);
    }
    check_launch();
    for (int b = 0; b < B; ++b)
      if (rows[b]) s->row_n[b] = 0;
  });
}

int rlt_set_batch_invariant(rlt_model* m, int on) {
  return guarded([&] {
    if (!m) fail(RLT_ERR_INVALID_ARG, "null model");
    m->batch_invariant = on ? 1 : 0;
  });
}

int rlt_state_block_steps(const rlt_state* s, int64_t* out) {
  return guarded([&] {
    if (!s || !out) fail(RLT_ERR_INVALID_ARG, "null state or output");
    *out = s->block_steps;
  });
}

int rlt_state_seek(rlt_model* m, rlt_state* s, int n, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (n < s->n_dec || n > s->n_enc) fail(RLT_ERR_ORDER, "seek target must lie between the decoded and encoded positions");
    const rlt_config& c = m->cfg;
    const int64_t ring = (int64_t)c.L_D * s->B * c.n_heads * s->R * c.d_head * (int64_t)m->esz;
    if (ring > 0) {
      fill_zero_u32(s->ring_k, ring / 4, stream);
      fill_zero_u32(s->ring_v, ring / 4, stream);
    }
    check_launch();
    s->n_dec = n;
  });
}

int rlt_set_scan_mode(rlt_model* m, int mode) {
  return guarded([&] {
    if (!m) fail(RLT_ERR_INVALID_ARG, "null model");
    if (mode < 0 || mode > 9) fail(RLT_ERR_INVALID_ARG, "scan mode must be 0..9");
    m->scan_mode = mode;
  });
}

int rlt_encode(rlt_model* m, rlt_state* s, const int32_t* tokens, int T, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (!tokens || T < 1) fail(RLT_ERR_INVALID_ARG, "tokens and T >= 1 required");
    if ((int64_t)s->n_enc + T > s->cap) fail(RLT_ERR_CAPACITY, "positions would exceed max_len");
    if (s->n_enc > 0 && !s->enc_k) fail(RLT_ERR_UNSUPPORTED, "continuing an encode needs keep_encoder_cache");
    do_encode(m, s, tokens, T, stream);
  });
}

int rlt_decode_scan(rlt_model* m, rlt_state* s, int T, float* logits, float* next_logprob,
                    const int32_t* next_tokens, float* s_out, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (T < 1) fail(RLT_ERR_INVALID_ARG, "T >= 1 required");
    if (next_logprob && !next_tokens) fail(RLT_ERR_INVALID_ARG, "next_logprob needs next_tokens");
    if ((int64_t)s->n_dec + T > s->n_enc) fail(RLT_ERR_ORDER, "decoder would pass the encoded positions");
    ScanOut o;
    o.logits = logits; o.ld_b = T; o.s_out = s_out;
    o.tok = next_tokens; o.tok_ld = T; o.lp = next_logprob; o.lp_ld = T;
    do_scan(m, s, T, o, stream);
  });
}

int rlt_step(rlt_model* m, rlt_state* s, const int32_t* tokens, float* logits, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (!tokens || !logits) fail(RLT_ERR_INVALID_ARG, "tokens and logits required");
    if (s->n_enc + 1 > s->cap) fail(RLT_ERR_CAPACITY, "positions would exceed max_len");
    if (s->n_enc > 0 && !s->enc_k) fail(RLT_ERR_UNSUPPORTED, "generation needs keep_encoder_cache");
    if (s->n_dec != s->n_enc) fail(RLT_ERR_ORDER, "consume the encoded positions before stepping");
    do_encode(m, s, tokens, 1, stream);
    ScanOut o;
    o.logits = logits; o.ld_b = 1;
    do_scan(m, s, 1, o, stream);
  });
}

int rlt_replay(rlt_model* m, rlt_state* s, const int32_t* tokens, int T, float* logprob, float* s_out,
               hipStream_t stream) {
  return guarded([&] {
    if (!m || !s || s->m != m) fail(RLT_ERR_INVALID_ARG, "null or foreign state");
    if (!tokens || T < 1) fail(RLT_ERR_INVALID_ARG, "tokens and T >= 1 required");
    if (T > s->cap) fail(RLT_ERR_CAPACITY, "T exceeds the state's max_len");
    if (rlt_state_reset(m, s, stream) != RLT_OK) fail(RLT_ERR_HIP, g_err);
    do_encode(m, s, tokens, T, stream);
    ScanOut o;
    o.ld_b = T;
    o.s_out = s_out;
    if (logprob && T > 1) {
      o.tok = tokens + 1; o.tok_ld = T;          // next token of position c+1 is tokens[b, c+1]
      o.lp = logprob; o.lp_ld = T - 1; o.lp_valid = T - 1;
    }
    do_scan(m, s, T, o, stream);
  });
}

int rlt_snapshot_size(rlt_model* m, rlt_state* s, int64_t* bytes) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (!bytes) fail(RLT_ERR_INVALID_ARG, "null output");
    *bytes = snapshot_payload(snapshot_parts(m, s, s->n_enc, s->n_dec, s->keep_enc != 0));
  });
}

int rlt_snapshot(rlt_model* m, rlt_state* s, void* dst, int64_t capacity, rlt_snapshot_info* info,
                 hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (!dst || !info) fail(RLT_ERR_INVALID_ARG, "dst and info required");
    const auto parts = snapshot_parts(m, s, s->n_enc, s->n_dec, s->keep_enc != 0);
    const int64_t need = snapshot_payload(parts);
    if (capacity < need) fail(RLT_ERR_CAPACITY, "snapshot buffer smaller than rlt_snapshot_size");
    snapshot_copy(parts, (char*)dst, false, stream);
    rlt_snapshot_info v{};
    v.config_digest = config_digest(m->cfg);
    v.weights_digest = m->wdigest;
    v.batch = s->B;
    v.n_encoded = s->n_enc;
    v.n_decoded = s->n_dec;
    v.window = m->cfg.window;
    v.ring_slots = s->R;
    v.has_encoder_cache = s->keep_enc;
    v.block_steps = s->block_steps;
    v.bytes = need;
    *info = v;
  });
}

int rlt_restore(rlt_model* m, rlt_state* s, const rlt_snapshot_info* info, const void* src, hipStream_t stream) {
  return guarded([&] {
    if (!m || !s || s->m != m) fail(RLT_ERR_INVALID_ARG, "null or foreign state");
    if (!info || !src) fail(RLT_ERR_INVALID_ARG, "info and src required");
    if (s->abort_host && *(volatile int*)s->abort_host)
      fail(RLT_ERR_HIP, "a persistent scan on this state timed out in a grid barrier; its results are invalid");
    if (info->config_digest != config_digest(m->cfg)) fail(RLT_ERR_INVALID_ARG, "snapshot of another configuration");
    if (info->weights_digest != m->wdigest)
      fail(RLT_ERR_STALE_STATE, "snapshot taken under other parameter values; recompute it from the tokens");
    if (info->batch != s->B) fail(RLT_ERR_INVALID_ARG, "snapshot batch differs from the state's");
    if (info->ring_slots != s->R || info->window != m->cfg.window)
      fail(RLT_ERR_INVALID_ARG, "snapshot ring layout differs from the state's");
    if (info->has_encoder_cache != s->keep_enc)
      fail(RLT_ERR_INVALID_ARG, "snapshot and state differ in keeping the encoder cache");
    if (info->n_encoded > s->cap) fail(RLT_ERR_CAPACITY, "snapshot positions exceed the state's max_len");
    if (info->n_decoded < 0 || info->n_decoded > info->n_encoded) fail(RLT_ERR_INVALID_ARG, "bad snapshot positions");
    const auto parts = snapshot_parts(m, s, info->n_encoded, info->n_decoded, s->keep_enc != 0);
    if (snapshot_payload(parts) != info->bytes) fail(RLT_ERR_INVALID_ARG, "snapshot size does not match its layout");
    snapshot_copy(parts, (char*)src, true, stream);
    check_launch();
    s->n_enc = info->n_encoded;
    s->n_dec = info->n_decoded;
    s->ragged = false;
    s->block_steps = info->block_steps;
    s->version = m->version;
  });
}

int rlt_sample_workspace(int rows, int vocab, int64_t* bytes) {
  return guarded([&] {
    if (!bytes || rows < 0 || vocab < 1) fail(RLT_ERR_INVALID_ARG, "rows >= 0, vocab >= 1 and bytes required");
    if (vocab > (1 << 20)) fail(RLT_ERR_UNSUPPORTED, "vocab > 2^20");
    *bytes = sample_workspace_bytes(rows, vocab);
  });
}

int rlt_sample(const float* logits, int rows, int vocab, int64_t ld, float temperature, uint64_t seed,
               uint64_t step, int32_t* tokens, float* logprob, void* workspace, int64_t workspace_bytes,
               hipStream_t stream) {
  return guarded([&] {
    if (!logits || !tokens) fail(RLT_ERR_INVALID_ARG, "logits and tokens required");
    if (rows < 0 || vocab < 1 || ld < vocab) fail(RLT_ERR_INVALID_ARG, "rows >= 0, vocab >= 1, ld >= vocab required");
    if (vocab > (1 << 20)) fail(RLT_ERR_UNSUPPORTED, "vocab > 2^20");
    if (!(temperature >= 0.f) || !std::isfinite(temperature))
      fail(RLT_ERR_INVALID_ARG, "temperature must be finite and >= 0");
    if (workspace && workspace_bytes < sample_workspace_bytes(rows, vocab))
      fail(RLT_ERR_INVALID_ARG, "workspace smaller than rlt_sample_workspace");
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15)) fail(RLT_ERR_INVALID_ARG, "workspace alignment");
    sample_rows(logits, ld, rows, vocab, temperature, seed, step, tokens, 1, logprob, 1, nullptr, stream, workspace);
    check_launch();
  });
}

int rlt_sample_noalloc(const float* logits, int rows, int vocab, int64_t ld, float temperature, uint64_t seed,
                       uint64_t step, int32_t* tokens, float* logprob, hipStream_t stream) {
  return guarded([&] {
    if (!logits || !tokens) fail(RLT_ERR_INVALID_ARG, "logits and tokens required");
    if (rows < 0 || vocab < 1 || ld < vocab) fail(RLT_ERR_INVALID_ARG, "rows >= 0, vocab >= 1, ld >= vocab required");
    if (vocab > (1 << 20)) fail(RLT_ERR_UNSUPPORTED, "vocab > 2^20");
    if (!(temperature >= 0.f) || !std::isfinite(temperature))
      fail(RLT_ERR_INVALID_ARG, "temperature must be finite and >= 0");
    if (sample_workspace_bytes(rows, vocab) > kSampleScratchBytes)
      fail(RLT_ERR_CAPACITY, "rows x vocabulary chunks exceed the static scratch (" +
                                 std::to_string(kSampleScratchBytes) + " bytes: rows * ceil(vocab / 4096) * 32)");
    void* ws = nullptr;
    HIPCHK(sample_scratch(&ws));
    sample_rows(logits, ld, rows, vocab, temperature, seed, step, tokens, 1, logprob, 1, nullptr, stream, ws);
    check_launch();
  });
}

int rlt_generate(rlt_model* m, rlt_state* s, const int32_t* first, int n, float temperature, uint64_t seed,
                 uint64_t step0, int32_t* tokens, float* logprob, float* logits, hipStream_t stream) {
  return guarded([&] {
    check_state(m, s);
    leave_ragged(s);
    if (!first || !tokens || !logprob) fail(RLT_ERR_INVALID_ARG, "first, tokens and logprob required");
    if (n < 1) fail(RLT_ERR_INVALID_ARG, "n >= 1 required");
    if (!(temperature >= 0.f) || !std::isfinite(temperature))
      fail(RLT_ERR_INVALID_ARG, "temperature must be finite and >= 0");
    if (s->n_enc + n > s->cap) fail(RLT_ERR_CAPACITY, "positions would exceed max_len");
    if (s->n_enc > 0 && !s->enc_k) fail(RLT_ERR_UNSUPPORTED, "generation needs keep_encoder_cache");
    if (s->n_dec != s->n_enc) fail(RLT_ERR_ORDER, "consume the encoded positions before generating");
    const int V = m->cfg.vocab;
    for (int i = 0; i < n; ++i) {
      // consume the last emitted token, then draw the next one from the new logits
      do_encode(m, s, i == 0 ? first : s->gtok, 1, stream);
      ScanOut o;
      o.logits = logits ? logits + (int64_t)i * V : s->glog;
      o.ld_b = logits ? n : 1;
      do_scan(m, s, 1, o, stream);
      sample_rows(o.logits, o.ld_b * V, s->B, V, temperature, seed, step0 + (uint64_t)i, tokens + i, n, logprob + i,
                  n, s->gtok, stream, s->samp_ws);
    }
    check_launch();
  });
}

int rlt_importance_ratio(const float* logprob_current, const float* logprob_behaviour, int64_t n, float* ratio,
                         hipStream_t stream) {
  return guarded([&] {
    if (n < 0) fail(RLT_ERR_INVALID_ARG, "n >= 0 required");
    if (n > 0 && (!logprob_current || !logprob_behaviour || !ratio)) fail(RLT_ERR_INVALID_ARG, "null pointer");
    importance_ratio(logprob_current, logprob_behaviour, n, ratio, stream);
    check_launch();
  });
}

int rlt_replay_grad_workspace(const rlt_config* cfg, int B, int T, int checkpoint, int64_t* bytes) {
  return guarded([&] {
    if (!cfg || !bytes) fail(RLT_ERR_INVALID_ARG, "null pointer");
    validate_config(*cfg);
    if (B < 1 || T < 2) fail(RLT_ERR_INVALID_ARG, "B >= 1 and T >= 2 required");
    *bytes = (int64_t)grad_workspace_bytes(*cfg, B, T, checkpoint != 0);
  });
}

int rlt_replay_grad(const rlt_config* cfg, const rlt_tensor* weights, int n_weights, rlt_grad_tensor* grads,
                    int n_grads, const int32_t* tokens, int B, int T, const float* dlogprob, float* logprob,
                    int checkpoint, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return guarded([&] {
    if (!cfg) fail(RLT_ERR_INVALID_ARG, "null config");
    validate_config(*cfg);
    if (B < 1 || T < 2) fail(RLT_ERR_INVALID_ARG, "B >= 1 and T >= 2 required");
    if (!tokens || !dlogprob || !logprob || !workspace) fail(RLT_ERR_INVALID_ARG, "null pointer");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) fail(RLT_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (workspace_bytes < (int64_t)grad_workspace_bytes(*cfg, B, T, checkpoint != 0))
      fail(RLT_ERR_INVALID_ARG, "workspace too small");
    auto W = index_weights(*cfg, weights, n_weights);
    if (n_grads < 0 || (n_grads > 0 && !grads)) fail(RLT_ERR_INVALID_ARG, "grads pointer");
    auto man = manifest(*cfg);
    std::map<std::string, std::pair<float*, int64_t>> G;
    for (int i = 0; i < n_grads; ++i) {
      if (!grads[i].name || !grads[i].data) fail(RLT_ERR_INVALID_ARG, "null gradient name or data");
      auto it = man.find(grads[i].name);
      if (it == man.end()) fail(RLT_ERR_INVALID_ARG, std::string("unknown gradient ") + grads[i].name);
      if (grads[i].numel != it->second.rows * it->second.cols)
        fail(RLT_ERR_INVALID_ARG, std::string("wrong size for gradient ") + grads[i].name);
      if (G.count(grads[i].name)) fail(RLT_ERR_INVALID_ARG, std::string("duplicate gradient ") + grads[i].name);
      G[grads[i].name] = {grads[i].data, grads[i].numel};
    }
    for (auto& kv : man)
      if (!G.count(kv.first)) fail(RLT_ERR_INVALID_ARG, "missing gradient " + kv.first);
    for (auto& kv : W)   // the products read weights as 16-byte vectors
      if (reinterpret_cast<uintptr_t>(kv.second) & 15) fail(RLT_ERR_INVALID_ARG, "weight " + kv.first + " not 16-byte aligned");
    hipError_t e = replay_grad(*cfg, W, G, tokens, B, T, dlogprob, logprob, workspace, checkpoint != 0, stream);
    if (e != hipSuccess) fail(RLT_ERR_HIP, std::string("replay gradient: ") + hipGetErrorString(e));
  });
}

}  // extern "C"
