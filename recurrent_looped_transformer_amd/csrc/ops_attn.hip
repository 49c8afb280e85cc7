// Attention of one query row per (sequence, head, query index) over a contiguous
// range of positions of a key/value store: the decoder's sliding-window
// self-attention over its ring (keys max(1, t-W+1)..t, greeksharifa summary
// §2.1, jiphyeonjeon review §3.3), the cross-attention to the prefix memory
// M_<=t (keys 1..t, greeksharifa summary §2.2, §2.4) and the encoder's
// attention over its cache.
//
// One workgroup (256 threads) per (head, query row). A group of DH/VEC lanes
// owns one key at a time (16-byte loads), so a wave reads whole contiguous key
// rows. Each group runs a single-pass online softmax over its keys, UNR keys per
// round; the K and V loads of the next round are issued before the current round
// computes (two register sets); the groups are combined through LDS at the end.
// Keys and values are each read once.
#include "common.hpp"
#include <algorithm>

#include "ops.hpp"

namespace rlt {

// SPLIT: this block takes the keys [z * split_keys, (z + 1) * split_keys) of its range
// (z = blockIdx.z) and writes its partial softmax sums to split_ws for attn_combine_k.
// X2: two-term query, keys and values (q_lo, kv_lo): each operand is hi + lo in fp32.
// NT: keys and values read with the nontemporal hint (launches that stream more than the
// last-level cache holds).
// NTH: threads per block (256; 512 when a launch leaves at least half the CUs without a block:
// twice the keys in flight per block — medium-LM decode, t 2048: B 8 2033 -> 1957 us per step,
// B 1 1575 -> 1548 us; at the paper shape, whose launches fill every CU, no faster).
template <typename T, int DH, bool SPLIT, int MEM, bool X2 = false, bool NT = false, int NTH = 256>
__global__ __launch_bounds__(NTH) void attn_decode_k(AttnArgs a) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int G = DH / VEC;              // lanes per key
  constexpr int NG = NTH / G;              // keys in flight per block per round
  constexpr int UNR = X2 ? 4 : 8;
  __shared__ float part[NG * DH];
  __shared__ float ml[2 * NG];
  const int h = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / a.nq, qi = row % a.nq;
  const int pos = (a.row_pos ? a.row_pos[b] : a.pos_dev ? a.pos_dev[0] : a.pos0) + 1 + qi;
  const int lo = a.window > 0 ? max(1, pos - a.window + 1) : 1;
  const int n = pos - lo + 1;
  const int tid = threadIdx.x, gi = tid / G, gl = tid % G;
  const int jb = SPLIT ? (int)blockIdx.z * a.split_keys : 0;
  const int je = SPLIT ? min(n, jb + a.split_keys) : n;

  // the query's raw bits now, unpacked after the first keys are requested (no wait in between)
  const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)row * a.ldq + h * DH + gl * VEC;
  const uint4 qraw = *reinterpret_cast<const uint4*>(qp);
  uint4 qraw_lo = make_uint4(0, 0, 0, 0);
  if constexpr (X2) qraw_lo = *reinterpret_cast<const uint4*>(qp + a.q_lo);
  const int64_t hb = (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH + gl * VEC;
  const T* kb = reinterpret_cast<const T*>(a.k) + hb;
  const T* vb = reinterpret_cast<const T*>(a.v) + hb;

  float m_run = -INFINITY, l_run = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  constexpr int STEP = NG * UNR;
  // software pipeline: the next round's keys and values are in flight while this round computes
  uint4 kk[UNR], vv[UNR], kn[UNR], vn[UNR];
  uint4 kkl[X2 ? UNR : 1], vvl[X2 ? UNR : 1], knl[X2 ? UNR : 1], vnl[X2 ? UNR : 1];
#define RLT_ATTN_LOAD(K_, V_, KL_, VL_, J0_)                                    \
  _Pragma("unroll") for (int u = 0; u < UNR; ++u) {                             \
    const int j = (J0_) + u * NG;                                               \
    if (j < je) {                                                               \
      const int p = lo + j;                                                     \
      const int slot = a.ring ? (p - 1) % a.cap : p - 1;                        \
      K_[u] = ld16<NT>(kb + (int64_t)slot * DH);                                \
      V_[u] = ld16<NT>(vb + (int64_t)slot * DH);                                \
      if constexpr (X2) {                                                       \
        KL_[u] = *reinterpret_cast<const uint4*>(kb + a.kv_lo + (int64_t)slot * DH); \
        VL_[u] = *reinterpret_cast<const uint4*>(vb + a.kv_lo + (int64_t)slot * DH); \
      }                                                                         \
    }                                                                           \
  }
  RLT_ATTN_LOAD(kk, vv, kkl, vvl, jb + gi)
  float qv[VEC];
  unpack16<T>(qraw, qv);
  if constexpr (X2) {
    float ql[VEC];
    unpack16<T>(qraw_lo, ql);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[e] += ql[e];
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] *= a.scale;
  for (int j0 = jb + gi; j0 < je; j0 += STEP) {
    if (j0 + STEP < je) RLT_ATTN_LOAD(kn, vn, knl, vnl, j0 + STEP)
    float sc[UNR];
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float dot = -INFINITY;
      if (j0 + u * NG < je) {
        float kf[VEC];
        unpack16<T>(kk[u], kf);
        if constexpr (X2) {
          float kl[VEC];
          unpack16<T>(kkl[u], kl);
#pragma unroll
          for (int e = 0; e < VEC; ++e) kf[e] += kl[e];
        }
        dot = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) dot = fmaf(qv[e], kf[e], dot);
      }
      dot = group_sum_dpp<G>(dot);
      sc[u] = dot;
      mx = fmaxf(mx, dot);
    }
    const float corr = __expf(m_run - mx);
    l_run *= corr;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= corr;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (j0 + u * NG < je) {
        const float pw = __expf(sc[u] - mx);
        l_run += pw;
        float vf[VEC];
        unpack16<T>(vv[u], vf);
        if constexpr (X2) {
          float vl[VEC];
          unpack16<T>(vvl[u], vl);
#pragma unroll
          for (int e = 0; e < VEC; ++e) vf[e] += vl[e];
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pw, vf[e], acc[e]);
      }
    }
    m_run = mx;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      kk[u] = kn[u];
      vv[u] = vn[u];
      if constexpr (X2) {
        kkl[u] = knl[u];
        vvl[u] = vnl[u];
      }
    }
  }
#undef RLT_ATTN_LOAD
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[gi * DH + gl * VEC + e] = acc[e];
  if (gl == 0) {
    ml[2 * gi] = m_run;
    ml[2 * gi + 1] = l_run;
  }
  __syncthreads();
  if (tid < DH) {
    float M = -INFINITY;
    for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, ml[2 * gg]);
    float s = 0.f, den = 0.f;
    if (!SPLIT || M != -INFINITY) {   // a split block past its row's last key has no keys
      for (int gg = 0; gg < NG; ++gg) {
        const float w = __expf(ml[2 * gg] - M);
        den += w * ml[2 * gg + 1];
        s += w * part[gg * DH + tid];
      }
    }
    if constexpr (SPLIT) {
      float* w = a.split_ws + (((int64_t)row * a.H + h) * gridDim.z + blockIdx.z) * (DH + 2);
      w[tid] = s;
      if (tid == 0) {
        w[DH] = M;
        w[DH + 1] = den;
      }
    } else {
      T* op = reinterpret_cast<T*>(a.out) + (int64_t)row * a.ldo + h * DH + tid;
      store_act<T>(op, a.out_split, s / den);
    }
  }
}

// Combines the key splits of attn_decode_k in ascending split order: out = sum_z e^(M_z - M)
// s_z / sum_z e^(M_z - M) den_z (empty splits carry M_z = -inf and weigh nothing).
template <typename T, int DH>
__global__ __launch_bounds__(DH) void attn_combine_k(AttnArgs a, int S) {
  const int h = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const float* w = a.split_ws + ((int64_t)row * a.H + h) * S * (DH + 2);
  float M = -INFINITY;
  for (int z = 0; z < S; ++z) M = fmaxf(M, w[z * (DH + 2) + DH]);
  float num = 0.f, den = 0.f;
  for (int z = 0; z < S; ++z) {
    const float mz = w[z * (DH + 2) + DH];
    if (mz == -INFINITY) continue;
    const float e = __expf(mz - M);
    num += e * w[z * (DH + 2) + tid];
    den += e * w[z * (DH + 2) + DH + 1];
  }
  T* op = reinterpret_cast<T*>(a.out) + (int64_t)row * a.ldo + h * DH + tid;
  store_act<T>(op, a.out_split, num / den);
}

template <typename T, int DH, int NTH>
static void launch_attn_variant(const AttnArgs& a, dim3 grid, int S, bool x2, bool nt, hipStream_t st) {
  const dim3 blk(NTH);
  if (S > 1) {
    if (x2) hipLaunchKernelGGL((attn_decode_k<T, DH, true, 0, true, false, NTH>), grid, blk, 0, st, a);
    else if (a.memory && nt) hipLaunchKernelGGL((attn_decode_k<T, DH, true, 1, false, true, NTH>), grid, blk, 0, st, a);
    else if (a.memory) hipLaunchKernelGGL((attn_decode_k<T, DH, true, 1, false, false, NTH>), grid, blk, 0, st, a);
    else if (nt) hipLaunchKernelGGL((attn_decode_k<T, DH, true, 0, false, true, NTH>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((attn_decode_k<T, DH, true, 0, false, false, NTH>), grid, blk, 0, st, a);
    hipLaunchKernelGGL((attn_combine_k<T, DH>), dim3(a.H, a.B * a.nq), dim3(DH), 0, st, a, S);
  } else {
    if (x2) hipLaunchKernelGGL((attn_decode_k<T, DH, false, 0, true, false, NTH>), grid, blk, 0, st, a);
    else if (a.memory && nt) hipLaunchKernelGGL((attn_decode_k<T, DH, false, 1, false, true, NTH>), grid, blk, 0, st, a);
    else if (a.memory) hipLaunchKernelGGL((attn_decode_k<T, DH, false, 1, false, false, NTH>), grid, blk, 0, st, a);
    else if (nt) hipLaunchKernelGGL((attn_decode_k<T, DH, false, 0, false, true, NTH>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((attn_decode_k<T, DH, false, 0, false, false, NTH>), grid, blk, 0, st, a);
  }
}

// Key splits: when the launch has at most kSplitMaxBlocks (head, query) blocks and its longest
// key range is long, every range is cut into pieces of split_keys keys (the same for every row,
// so a long prefix gets more blocks than a short one), one round of at most 256 blocks in
// all; the pieces are combined by attn_combine_k. Measured on the medium-LM decode (16
// heads, dh 128, t 2048): 8 rows split 16 ways ran 6.7 us slower per launch than unsplit (the
// extra launch and per-block overheads outweigh the occupancy), so launches of more than
// kSplitMaxBlocks blocks split only into pieces of at least kSplitLongPiece keys, when they
// would otherwise leave CUs idle (paper shape, 32 heads, t 8192: 2 rows unsplit streamed the
// memory at 2.9 TB/s on 64 blocks, 4 rows at 5.0 TB/s on 128).
constexpr int kSplitMinKeys = 1024, kSplitMaxBlocks = 32, kSplitPiece = 256, kSplitRound = 256,
              kSplitLongPiece = 2048;
static_assert(kSplitRound <= kAttnSplitBlocks, "split workspace");
template <typename T, int DH>
static void launch_attn(const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  const int blocks = a.H * a.B * a.nq;
  int S = 1;
  if (a.split_ws && a.n_max >= kSplitMinKeys && blocks < kSplitRound) {
    S = std::min({(a.n_max + kSplitPiece - 1) / kSplitPiece, kSplitRound / blocks, a.split_max});
    if (blocks > kSplitMaxBlocks) S = std::min(S, a.n_max / kSplitLongPiece);
    S = std::max(S, 1);
    a.split_keys = (a.n_max + S - 1) / S;
    S = (a.n_max + a.split_keys - 1) / a.split_keys;
  }
  // the memory attention runs its own instance of the same code (MEM = 1): a separate symbol;
  // two-term operands (the encoder's, 16-bit types) take the X2 instances. Launches of at most
  // 128 blocks take blocks of 512 threads when the caller allows it (not in batch-invariant
  // mode: a row's arithmetic must not depend on the batch)
  const dim3 grid(a.H, a.B * a.nq, S);
  const bool x2 = !__is_same(T, float) && (a.q_lo > 0 || a.kv_lo > 0);
  const bool nt = a.stream != 0 && !x2;
  const bool wide = DH >= 64 && a.wide && (int64_t)grid.x * grid.y * grid.z <= 128;
  if (wide) launch_attn_variant<T, DH, 512>(a, grid, S, x2, nt, st);
  else launch_attn_variant<T, DH, 256>(a, grid, S, x2, nt, st);
}

template <typename T>
static void attn_dispatch(const AttnArgs& a, hipStream_t st) {
  switch (a.dh) {
    case 16: launch_attn<T, 16>(a, st); break;
    case 32: launch_attn<T, 32>(a, st); break;
    case 64: launch_attn<T, 64>(a, st); break;
    case 128: launch_attn<T, 128>(a, st); break;
    case 256: launch_attn<T, 256>(a, st); break;
    default: break;   // rejected on the host
  }
}

void attn_decode(Dt dt, const AttnArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.nq <= 0) return;
  if (dt == Dt::F32) attn_dispatch<float>(a, st);
  else if (dt == Dt::BF16) attn_dispatch<bf16_t>(a, st);
  else attn_dispatch<f16_t>(a, st);
}

}  // namespace rlt

// ====================================================================== prefill
// Causal (optionally windowed) attention of many queries per (sequence, head) with
// bf16 MFMA, flash style: the encoder's token-parallel self-attention
// (greeksharifa summary §2.2: each encoder layer processes the given positions
// together under a causal mask).
//
// Block = 4 waves = 256 queries at dh 64 (64 per wave, as 4 MFMA column blocks of 16; 128
// queries as 2 blocks of 16 per wave at dh 128) of one (sequence, head); keys and values stream through LDS in tiles of 64 positions, double
// buffered (the next tile's loads are in registers while the current one computes; V is
// stored transposed, 4 keys per 8-byte write). Each wave computes S^T = K Q^T with 16x16x32
// MFMAs: lane l then holds the scores of 4 keys of query l % 16. Key rows sit in LDS in a
// permuted order (LDS row 32 p + 16 h + 4 a + i holds key 32 p + 8 a + 4 h + i), so that over
// two adjacent 16-key sub-tiles lane l holds keys 8g..8g+7 (g = l / 16) of a 32-key half: exactly
// the B operand of the 16x16x32 MFMA for O^T += V^T P^T, so probabilities never leave
// registers, and the weighted sum takes one product per 32 keys (two 16x16x16 products issue
// at half the rate on this part). Each K or V^T fragment read from LDS feeds the query blocks
// of the wave. Softmax statistics are fp32 per query, online over key tiles, in base 2 with
// log2(e) folded into the score scale; tiles that every query of a wave sees whole skip the mask.
namespace rlt {

// QB query blocks of 16 per wave: up to 4 (2 for bf16 at dh 128: register budget); short
// sequences take one so that the grid keeps enough workgroups.
// Row pitches: KP = DH / 8 + 1 uint4 per K row (the 16 rows a fragment read touches start 4
// banks apart); VP = BK + 4 halves per V^T row (136 bytes: the 16 rows of a PV fragment read
// start 34 banks apart, distinct bank pairs — a pitch of 72 put rows c and c + 8 on one pair).
template <typename T, int DH, int QB>
__global__ __launch_bounds__(256) void flash_prefill_k(AttnArgs a) {
  constexpr int BK = 64, KP = DH / 8 + 1, VP = BK + 4, QW = 16 * QB, QBLK = 4 * QW;
  constexpr int PARTS = DH / 8;                      // 16-byte chunks of a key row
  constexpr int LOADERS = 16 * PARTS;                // threads that stage a tile: 4 keys x 8 values each
  __shared__ __align__(16) uint4 sK[2][BK][KP];
  __shared__ __align__(16) uint16_t sVt[2][DH][VP];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int g = lane >> 4, c = lane & 15;
  const int q0 = qb * QBLK + wave * QW;              // first query (within this call) of the wave
  uint4 qf[QB][DH / 32];
  int qpos[QB];
  bool qvalid[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int myq = q0 + j * 16 + c;
    qvalid[j] = myq < a.nq;
    qpos[j] = a.pos0 + 1 + myq;
    const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.nq + min(myq, a.nq - 1)) * a.ldq +
                        h * DH;
#pragma unroll
    for (int kc = 0; kc < DH / 32; ++kc) qf[j][kc] = *reinterpret_cast<const uint4*>(Q + kc * 32 + g * 8);
  }
  f32x4 o[QB][DH / 16];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) o[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }
  const float scale2 = a.scale * 1.4426950408889634f;     // scores in base 2
  const int qlast = min(a.nq, (qb + 1) * QBLK);        // queries of this block: [qb*QBLK, qlast)
  const int kmax = a.pos0 + qlast;                       // last key position any query here needs
  const int kmin = a.window > 0 ? max(1, a.pos0 + 1 + qb * QBLK - a.window + 1) : 1;
  const bool wave_full_q = q0 + QW <= a.nq;              // the wave's queries all valid
  const int wq_first = a.pos0 + 1 + q0, wq_last = a.pos0 + q0 + QW;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH;

  // staging: thread t < LOADERS owns keys 4 jq .. 4 jq + 3 (jq = t / PARTS), 16-byte chunk part
  // of K, and keys 4 jv .. 4 jv + 3 (jv = t % 16), chunk pv = t / 16 of V: the V^T writes of
  // a wave then spread over every LDS bank (with the K mapping, the 16 chunks of a wave's
  // rows fell on two bank groups: 8-way conflicts)
  const int jq = tid / PARTS, part = tid % PARTS;
  const int jv = tid % 16, pv = tid / 16;
  // LDS row of key 4 jq in the permuted key order described above
  const int krow = 32 * (jq >> 3) + 16 * (jq & 1) + 4 * ((jq >> 1) & 3);
  uint4 rk[4], rv[4];
  // positions past kmax load the row of kmax (valid data: their scores are masked, so they
  // weigh zero); a ring slot is the tile's first slot (one scalar modulo) plus the key's
  // offset, wrapped once (the launch guarantees cap >= BK)
  // (the staging registers are defined on every path: otherwise they are kept in scratch)
  auto gload = [&](int k0) {
    const int s0 = a.ring ? (k0 - 1) % a.cap : k0 - 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rk[e] = make_uint4(0, 0, 0, 0);
      rv[e] = make_uint4(0, 0, 0, 0);
    }
    if (tid < LOADERS) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int sp = s0 + min(4 * jq + e, kmax - k0), sq = s0 + min(4 * jv + e, kmax - k0);
        if (a.ring) {
          sp = sp >= a.cap ? sp - a.cap : sp;
          sq = sq >= a.cap ? sq - a.cap : sq;
        }
        rk[e] = *reinterpret_cast<const uint4*>(Kb + (int64_t)sp * DH + part * 8);
        rv[e] = *reinterpret_cast<const uint4*>(Vb + (int64_t)sq * DH + pv * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
    if (tid < LOADERS) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sK[buf][krow + e][part] = rk[e];
      const uint32_t w[4][4] = {{rv[0].x, rv[0].y, rv[0].z, rv[0].w}, {rv[1].x, rv[1].y, rv[1].z, rv[1].w},
                                {rv[2].x, rv[2].y, rv[2].z, rv[2].w}, {rv[3].x, rv[3].y, rv[3].z, rv[3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {   // value e of the chunk for the 4 keys: one 8-byte write of V^T
        const int sh = (e & 1) * 16;
        uint2 t;
        t.x = ((w[0][e >> 1] >> sh) & 0xffffu) | (((w[1][e >> 1] >> sh) & 0xffffu) << 16);
        t.y = ((w[2][e >> 1] >> sh) & 0xffffu) | (((w[3][e >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&sVt[buf][pv * 8 + e][4 * jv]) = t;
      }
    }
  };

  gload(kmin);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kmin; k0 <= kmax; k0 += BK) {
    const bool more = k0 + BK <= kmax;
    if (more) gload(k0 + BK);
    __builtin_amdgcn_sched_barrier(0);   // the next tile's loads stay ahead of this tile's work
    const bool whole = wave_full_q && k0 + BK - 1 <= wq_first && (a.window <= 0 || k0 > wq_last - a.window);
    // all score products first (no branch between them), then the mask
    f32x4 sacc[QB][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 kf[DH / 32];
#pragma unroll
      for (int kc = 0; kc < DH / 32; ++kc) kf[kc] = sK[buf][st * 16 + c][kc * 4 + g];
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < DH / 32; ++kc) acc = mfma16x16x32<T>(kf[kc], qf[j][kc], acc);
        sacc[j][st] = acc;
      }
    }
    float s[QB][4][4];
    float tmax[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) tmax[j] = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const f32x4 acc = sacc[j][st];
        if (whole) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[j][st][i] = acc[i] * scale2;
            tmax[j] = fmaxf(tmax[j], s[j][st][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kp = k0 + 32 * (st >> 1) + 8 * g + 4 * (st & 1) + i;   // permuted key rows
            const bool ok =
                qvalid[j] && kp <= qpos[j] && kp <= kmax && (a.window <= 0 || kp > qpos[j] - a.window);
            s[j][st][i] = ok ? acc[i] * scale2 : -INFINITY;
            tmax[j] = fmaxf(tmax[j], s[j][st][i]);
          }
        }
      }
    }
    uint4 pb[QB][2];                             // [query block][32-key half]: keys 8 g .. 8 g + 7
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float tm = fmaxf(tmax[j], __shfl_xor(tmax[j], 16, WAVE));
      tm = fmaxf(tm, __shfl_xor(tm, 32, WAVE));
      const float m_new = fmaxf(m_run[j], tm);
      // branch-free: a column with nothing visible yet keeps l = 0 and o = 0 (exp(-inf) = 0)
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __builtin_amdgcn_exp2f(m_run[j] - m_use);
      l_run[j] *= corr;
#pragma unroll
      for (int i = 0; i < DH / 16; ++i) o[j][i] *= corr;
      float lsum = 0.f;
      uint32_t w[4][2];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(s[j][st][i] - m_use);
          lsum += pv[i];
        }
        w[st][0] = pack2<T>(pv[0], pv[1]);
        w[st][1] = pack2<T>(pv[2], pv[3]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) pb[j][p] = make_uint4(w[2 * p][0], w[2 * p][1], w[2 * p + 1][0], w[2 * p + 1][1]);
      lsum += __shfl_xor(lsum, 16, WAVE);
      lsum += __shfl_xor(lsum, 32, WAVE);
      l_run[j] += lsum;
      m_run[j] = m_new;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) {
        const uint16_t* r0 = &sVt[buf][db * 16 + c][p * 32 + 8 * g];
        const uint2 v0 = *reinterpret_cast<const uint2*>(r0), v1 = *reinterpret_cast<const uint2*>(r0 + 4);
        const uint4 av = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int j = 0; j < QB; ++j) o[j][db] = mfma16x16x32<T>(av, pb[j][p], o[j][db]);
      }
    }
    if (more) lstore(buf ^ 1);   // buffer buf ^ 1 was last read before the previous barrier
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (!qvalid[j]) continue;
    const int myq = q0 + j * 16 + c;
    const float inv = l_run[j] > 0.f ? 1.f / l_run[j] : 0.f;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.nq + myq) * a.ldo + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
      float v[4] = {o[j][db][0] * inv, o[j][db][1] * inv, o[j][db][2] * inv, o[j][db][3] * inv};
      uint2 w;
      w.x = pack2<T>(v[0], v[1]);
      w.y = pack2<T>(v[2], v[3]);
      *reinterpret_cast<uint2*>(out + db * 16 + 4 * g) = w;
      if (a.out_split) {   // lo terms
        uint2 l;
        l.x = pack2<T>(v[0] - Elem<T>::round(v[0]), v[1] - Elem<T>::round(v[1]));
        l.y = pack2<T>(v[2] - Elem<T>::round(v[2]), v[3] - Elem<T>::round(v[3]));
        *reinterpret_cast<uint2*>(out + a.out_split + db * 16 + 4 * g) = l;
      }
    }
  }
}

// Two-term operands (q_lo, kv_lo > 0): every query, key and value is hi + lo in the 16-bit
// type. (This kernel keeps key rows in natural order and the 16x16x16 weighted sum: the key
// permutation, 16x16x32 weighted sum and whole-tile path of the one-term kernel cut its
// MFMA-busy cycles by a third but measured 1.2% slower on the paper-shape encode and no faster
// on the medium-LM encode; its time is not set by the MFMA count.) Scores take three MFMA
// products (K_hi Q_hi + K_hi Q_lo + K_lo Q_hi; the lo * lo term is
// below the fp32 rounding of the sum), the probabilities are split into hi + lo in registers
// and the weighted sum takes V_hi P_hi + V_hi P_lo + V_lo P_hi. Same tiling as above with both
// terms of a key / value tile in LDS (4 stages: buffer x term); at most two query blocks per
// wave (register budget).
template <typename T, int DH, int QB, int NW = 4>
__global__ __launch_bounds__(NW * WAVE) void flash_prefill_x2_k(AttnArgs a) {
  constexpr int BK = 64, KP = DH / 8 + 1, VP = BK + 4, QW = 16 * QB, QBLK = NW * QW;
  constexpr int PARTS = DH / 8;
  constexpr int LOADERS = 16 * PARTS;
  __shared__ __align__(16) uint4 sK[2][2][BK][KP];           // [buffer][term]
  __shared__ __align__(16) uint16_t sVt[2][2][DH][VP];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int g = lane >> 4, c = lane & 15;
  const int q0 = qb * QBLK + wave * QW;
  uint4 qh[QB][DH / 32], ql[QB][DH / 32];
  int qpos[QB];
  bool qvalid[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int myq = q0 + j * 16 + c;
    qvalid[j] = myq < a.nq;
    qpos[j] = a.pos0 + 1 + myq;
    const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.nq + min(myq, a.nq - 1)) * a.ldq +
                        h * DH;
#pragma unroll
    for (int kc = 0; kc < DH / 32; ++kc) {
      qh[j][kc] = *reinterpret_cast<const uint4*>(Q + kc * 32 + g * 8);
      ql[j][kc] = *reinterpret_cast<const uint4*>(Q + a.q_lo + kc * 32 + g * 8);
    }
  }
  f32x4 o[QB][DH / 16];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) o[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }
  const int qlast = min(a.nq, (qb + 1) * QBLK);
  const int kmax = a.pos0 + qlast;
  const int kmin = a.window > 0 ? max(1, a.pos0 + 1 + qb * QBLK - a.window + 1) : 1;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH;
  const uint16_t* Vb = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH;

  // K and V staged by different thread mappings (see flash_prefill_k): conflict-free V^T writes
  const int jq = tid / PARTS, part = tid % PARTS;
  const int jv = tid % 16, pv = tid / 16;
  uint4 rk[2][4], rv[2][4];                                   // [term][key]
  auto gload = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = k0 + 4 * jq + e, q = k0 + 4 * jv + e;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        rk[t][e] = make_uint4(0, 0, 0, 0);
        rv[t][e] = make_uint4(0, 0, 0, 0);
      }
      if (tid < LOADERS && p <= kmax) {
        const int slot = a.ring ? (p - 1) % a.cap : p - 1;
        const int64_t off = (int64_t)slot * DH + part * 8;
        rk[0][e] = *reinterpret_cast<const uint4*>(Kb + off);
        rk[1][e] = *reinterpret_cast<const uint4*>(Kb + a.kv_lo + off);
      }
      if (tid < LOADERS && q <= kmax) {
        const int slot = a.ring ? (q - 1) % a.cap : q - 1;
        const int64_t off = (int64_t)slot * DH + pv * 8;
        rv[0][e] = *reinterpret_cast<const uint4*>(Vb + off);
        rv[1][e] = *reinterpret_cast<const uint4*>(Vb + a.kv_lo + off);
      }
    }
  };
  auto lstore = [&](int buf) {
    if (tid < LOADERS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sK[buf][t][4 * jq + e][part] = rk[t][e];
        const uint32_t w[4][4] = {{rv[t][0].x, rv[t][0].y, rv[t][0].z, rv[t][0].w},
                                  {rv[t][1].x, rv[t][1].y, rv[t][1].z, rv[t][1].w},
                                  {rv[t][2].x, rv[t][2].y, rv[t][2].z, rv[t][2].w},
                                  {rv[t][3].x, rv[t][3].y, rv[t][3].z, rv[t][3].w}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          uint2 u;
          u.x = ((w[0][e >> 1] >> sh) & 0xffffu) | (((w[1][e >> 1] >> sh) & 0xffffu) << 16);
          u.y = ((w[2][e >> 1] >> sh) & 0xffffu) | (((w[3][e >> 1] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<uint2*>(&sVt[buf][t][pv * 8 + e][4 * jv]) = u;
        }
      }
    }
  };

  gload(kmin);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = kmin; k0 <= kmax; k0 += BK) {
    const bool more = k0 + BK <= kmax;
    if (more) gload(k0 + BK);
    float s[QB][4][4];
    float tmax[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) tmax[j] = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 kh[DH / 32], kl[DH / 32];
#pragma unroll
      for (int kc = 0; kc < DH / 32; ++kc) {
        kh[kc] = sK[buf][0][st * 16 + c][kc * 4 + g];
        kl[kc] = sK[buf][1][st * 16 + c][kc * 4 + g];
      }
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < DH / 32; ++kc) {
          acc = mfma16x16x32<T>(kl[kc], qh[j][kc], acc);
          acc = mfma16x16x32<T>(kh[kc], ql[j][kc], acc);
          acc = mfma16x16x32<T>(kh[kc], qh[j][kc], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kp = k0 + st * 16 + 4 * g + i;
          const bool ok = qvalid[j] && kp <= qpos[j] && kp <= kmax && (a.window <= 0 || kp > qpos[j] - a.window);
          s[j][st][i] = ok ? acc[i] * a.scale : -INFINITY;
          tmax[j] = fmaxf(tmax[j], s[j][st][i]);
        }
      }
    }
    uint2 pbh[QB][4], pbl[QB][4];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      float tm = fmaxf(tmax[j], __shfl_xor(tmax[j], 16, WAVE));
      tm = fmaxf(tm, __shfl_xor(tm, 32, WAVE));
      const float m_new = fmaxf(m_run[j], tm);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __expf(m_run[j] - m_use);
      l_run[j] *= corr;
#pragma unroll
      for (int i = 0; i < DH / 16; ++i) o[j][i] *= corr;
      float lsum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __expf(s[j][st][i] - m_use);
          lsum += pv;
          ph[i] = Elem<T>::round(pv);
          pl[i] = pv - ph[i];
        }
        pbh[j][st].x = pack2<T>(ph[0], ph[1]);
        pbh[j][st].y = pack2<T>(ph[2], ph[3]);
        pbl[j][st].x = pack2<T>(pl[0], pl[1]);
        pbl[j][st].y = pack2<T>(pl[2], pl[3]);
      }
      lsum += __shfl_xor(lsum, 16, WAVE);
      lsum += __shfl_xor(lsum, 32, WAVE);
      l_run[j] += lsum;
      m_run[j] = m_new;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) {
        const uint2 vh = *reinterpret_cast<const uint2*>(&sVt[buf][0][db * 16 + c][st * 16 + 4 * g]);
        const uint2 vl = *reinterpret_cast<const uint2*>(&sVt[buf][1][db * 16 + c][st * 16 + 4 * g]);
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          o[j][db] = mfma16x16x16<T>(vl, pbh[j][st], o[j][db]);
          o[j][db] = mfma16x16x16<T>(vh, pbl[j][st], o[j][db]);
          o[j][db] = mfma16x16x16<T>(vh, pbh[j][st], o[j][db]);
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    if (!qvalid[j]) continue;
    const int myq = q0 + j * 16 + c;
    const float inv = l_run[j] > 0.f ? 1.f / l_run[j] : 0.f;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.nq + myq) * a.ldo + h * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) {
      float v[4] = {o[j][db][0] * inv, o[j][db][1] * inv, o[j][db][2] * inv, o[j][db][3] * inv};
      uint2 w;
      w.x = pack2<T>(v[0], v[1]);
      w.y = pack2<T>(v[2], v[3]);
      *reinterpret_cast<uint2*>(out + db * 16 + 4 * g) = w;
      if (a.out_split) {
        uint2 l;
        l.x = pack2<T>(v[0] - Elem<T>::round(v[0]), v[1] - Elem<T>::round(v[1]));
        l.y = pack2<T>(v[2] - Elem<T>::round(v[2]), v[3] - Elem<T>::round(v[3]));
        *reinterpret_cast<uint2*>(out + a.out_split + db * 16 + 4 * g) = l;
      }
    }
  }
}

template <typename T, int DH>
static void launch_flash(const AttnArgs& a, hipStream_t st) {
  if (a.q_lo > 0 || a.kv_lo > 0) {
    if (a.nq <= 512) {
      hipLaunchKernelGGL((flash_prefill_x2_k<T, DH, 1>), dim3((a.nq + 63) / 64, a.H, a.B), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((flash_prefill_x2_k<T, DH, 1, 8>), dim3((a.nq + 127) / 128, a.H, a.B), dim3(512), 0, st, a);
    }
    return;
  }
  // four query blocks per wave; at dh 128 fp16 that is 1.3x over two at the medium-LM encode
  // (measured; 256 + 256 registers, no spills), while bf16 (whose unpacking takes more
  // registers) would spill there and keeps two
  constexpr int QBMAX = (DH >= 128 && !__is_same(T, f16_t)) ? 2 : 4;
  if (a.nq <= 512) {
    hipLaunchKernelGGL((flash_prefill_k<T, DH, 1>), dim3((a.nq + 63) / 64, a.H, a.B), dim3(256), 0, st, a);
  } else {
    const int qblk = 64 * QBMAX;
    hipLaunchKernelGGL((flash_prefill_k<T, DH, QBMAX>), dim3((a.nq + qblk - 1) / qblk, a.H, a.B), dim3(256), 0, st,
                       a);
  }
}

bool attn_prefill(Dt dt, const AttnArgs& a, hipStream_t st) {
  if ((a.dh != 64 && a.dh != 128) || dt == Dt::F32) return false;
  if (a.ring && a.cap < 64) return false;   // a tile's ring slots wrap at most once
  if (dt == Dt::BF16) {
    if (a.dh == 64) launch_flash<bf16_t, 64>(a, st);
    else launch_flash<bf16_t, 128>(a, st);
  } else {
    if (a.dh == 64) launch_flash<f16_t, 64>(a, st);
    else launch_flash<f16_t, 128>(a, st);
  }
  return true;
}

}  // namespace rlt
