// Persistent decoder-scan kernel (one cooperative launch per scan).
//
// The scan is the sequential part of the method: every consumed position runs
// the merge and the L_D decoder blocks, batched over the B independent
// sequences (greeksharifa summary §2.3-§2.7; jiphyeonjeon review §3.3,
// eq 2.9-2.16, §5 / Figure 3: batch the next update of independent sequences).
// A pass handles np positions (1 for RLT-1, one chunk for RLT-2, up to P
// parallel positions for RLT-0); rows are m = b * np + i.
//
// Phases of a pass (grid-wide barrier after each):
//   MERGE/INIT  u = e + alpha*sigmoid(gpre + W_g,r r)*(W_s r)  (RLT-0: u = e),
//               plus the row copies that finish the previous pass
//   per layer:  QKV(+RoPE, ring write) | SWA | O(+res) | Xq(+RoPE) | CROSS | Xo(+res) | W13(SwiGLU) | W2(+res)
//   FINAL       row copies of the last pass
// RMSNorm is folded into the producers: every residual update writes z (fp32),
// zb = bf16(z * gain of the next norm) and per-16-feature sums of squares; the
// consuming GEMM multiplies its accumulator by rsqrt(mean(z^2) + eps).
//
// Cross-workgroup data (z, zb, sum-of-squares partials, q, attention outputs,
// SwiGLU hidden, ring K/V, register) is stored and loaded with device-scope
// (SC1) buffer instructions, so visibility needs only s_waitcnt before the
// barrier and never an L2 writeback / invalidate. Weights, encoder outputs and
// memory are written before the launch and read with ordinary loads.
#include "ops.hpp"
#include "scan.hpp"

namespace rlt {

typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int SC1 = 16;          // cache-policy bit: device scope
constexpr int V0_ = 0, V2_ = 2;

// Buffer descriptor of a workgroup-uniform base pointer. The pointer is made provably
// uniform (readfirstlane) so the descriptor lives in scalar registers; every caller passes
// a pointer that is the same for all lanes of the workgroup.
__device__ __forceinline__ Rsrc mk(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, -1, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16c(Rsrc r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1); }
__device__ __forceinline__ u32 ld4c(Rsrc r, u32 off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1); }
__device__ __forceinline__ void st16c(Rsrc r, u32 off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC1); }
__device__ __forceinline__ void st8c(Rsrc r, u32 off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, SC1); }
__device__ __forceinline__ void st4c(Rsrc r, u32 off, u32 v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, SC1); }
__device__ __forceinline__ float ldf_c(Rsrc r, u32 off) { return __uint_as_float(ld4c(r, off)); }

__device__ __forceinline__ u32 pack2(float a, float b) { return (u32)f2bf(a) | ((u32)f2bf(b) << 16); }
__device__ __forceinline__ void unpack8(u32x4 v, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(v[i] << 16);
    o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// ------------------------------------------------------------------ barriers
// Words (u32 index): per-XCD arrival counters at 64*x (x < 8), top counter 64*8,
// release flag 64*9, abort 64*10, member flags of group g at 64*(16+g) + k.
__device__ __forceinline__ u32 aload(u32* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u32 aadd(u32* p, u32 v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void astore(u32* p, u32 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
constexpr long kSpinLimit = 1l << 22;

// Whole grid: arrivals counted per XCD (blocks are dealt to XCDs round robin), the last
// arrival of each XCD bumps a top counter, the last of those releases everyone.
__device__ __noinline__ bool grid_sync(u32* bar, u32& epoch, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's device-scope stores are complete
  __syncthreads();
  epoch += 1;
  if (threadIdx.x == 0) {
    const int nb = gridDim.x;
    const int ng = nb < 8 ? nb : 8;
    const int x = blockIdx.x % ng;
    const u32 per = (u32)((nb - x + ng - 1) / ng);
    int ok = 1;
    const u32 old = aadd(&bar[64 * x], 1u);
    if (old == epoch * per - 1) {
      const u32 o2 = aadd(&bar[64 * 8], 1u);
      if (o2 == epoch * (u32)ng - 1) astore(&bar[64 * 9], epoch);
    }
    long spins = 0;
    while (aload(&bar[64 * 9]) < epoch) {
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 63) == 0 && aload(&bar[64 * 10])) { ok = 0; break; }
      if (spins > kSpinLimit) { astore(&bar[64 * 10], 1u); ok = 0; break; }
    }
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

// One group (the blocks of one XCD): each member publishes its epoch in its own
// word; the first wave polls all members' words.
__device__ __noinline__ bool group_sync(u32* bar, u32& epoch, int* s_flag, int grp, int rank, int nmem) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  epoch += 1;
  if (threadIdx.x < WAVE) {
    u32* flags = bar + 64 * (16 + grp);
    if (threadIdx.x == 0) astore(&flags[rank], epoch);
    int ok = 1;
    long spins = 0;
    while (true) {
      u32 v = threadIdx.x < (unsigned)nmem ? aload(&flags[threadIdx.x]) : 0xffffffffu;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v = min(v, (u32)__shfl_xor((int)v, o, WAVE));
      if (v >= epoch) break;
      if ((++spins & 63) == 0 && aload(&bar[64 * 10])) { ok = 0; break; }
      if (spins > kSpinLimit) { if (threadIdx.x == 0) astore(&bar[64 * 10], 1u); ok = 0; break; }
    }
    if (threadIdx.x == 0) *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

// ------------------------------------------------------------------ GEMM tile
// Weights of one 16-row tile for the first two 64-wide K chunks of this wave
// (c = wave, wave + 4); loaded before the barrier that precedes the GEMM phase,
// since weights never depend on it.
struct WPre {
  uint4 a[2][2];
};
__device__ __forceinline__ void w_prefetch(WPre& w, const bf16_t* __restrict__ W, int N, int K, int n0) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const bf16_t* wp = W + (int64_t)(n0 >> 4) * 16 * K + lane * 8;   // tile-major weight tile
  const int nch = K / 64;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int cc = wave + 4 * u;
    if (cc < nch) {
      w.a[u][0] = *reinterpret_cast<const uint4*>(wp + cc * 1024);
      w.a[u][1] = *reinterpret_cast<const uint4*>(wp + cc * 1024 + 512);
    }
  }
}

// acc for weight rows n0..n0+15 (plain loads from the tile-major W) and activation rows
// m0 + 16 j + r (device-scope loads from X with leading dimension ldx at buffer row
// xrow(m) = (m / q) * xp + m % q + xo), j < nmb, rows limited to [.., M). Waves split
// K in chunks of 64; each wave issues the loads of two chunks before their MFMAs; the
// first two chunks' weights come from `pre` when given. Partial sums go to red; the
// caller reduces them after a block barrier (tile_sum).
__device__ __forceinline__ void tile_mma(const bf16_t* __restrict__ W, int N, int K, int n0, Rsrc xr, int ldx, int q,
                                         int xp, int xo, int M, int m0, int nmb, f32x4 (*red)[4][WAVE],
                                         const WPre* pre = nullptr) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r = lane & 15, g = lane >> 4;
  const bf16_t* wp = W + (int64_t)(n0 >> 4) * 16 * K + lane * 8;   // tile-major weight tile
  u32 xoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mm = min(m0 + j * 16 + r, M - 1);
    xoff[j] = (u32)(((int64_t)(mm / q) * xp + mm % q + xo) * ldx + g * 16) * 2u;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = K / 64;
  for (int c = wave; c < nch; c += 8) {
    const bool two = c + 4 < nch;
    uint4 a[2][2], b[2][4][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 0 || two) {
        const int cc = c + 4 * u;
        if (pre && c == wave) {
          a[u][0] = pre->a[u][0];
          a[u][1] = pre->a[u][1];
        } else {
          a[u][0] = *reinterpret_cast<const uint4*>(wp + cc * 1024);
          a[u][1] = *reinterpret_cast<const uint4*>(wp + cc * 1024 + 512);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < nmb) {
            b[u][j][0] = as_uint4(ld16c(xr, xoff[j] + cc * 128));
            b[u][j][1] = as_uint4(ld16c(xr, xoff[j] + cc * 128 + 16));
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 0 || two) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < nmb) {
            acc[j] = mfma16x16x32(a[u][0], b[u][j][0], acc[j]);
            acc[j] = mfma16x16x32(a[u][1], b[u][j][1], acc[j]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][j][lane] = acc[j];
}

// after a barrier: the reduced tile of m-block `wave`
__device__ __forceinline__ f32x4 tile_sum(int nmb, f32x4 (*red)[4][WAVE]) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < nmb) s = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
  return s;
}

// Row RMS factors rs[i] = rsqrt(sum_t ssp[t * ld + xrow(m0 + i)] / d + eps), i < 64 (rows
// beyond M get 1), xrow(m) = (m / q) * xp + m % q + xo. rms_issue starts the loads (four
// threads per row, up to 16 partials each); rms_finish sums them in a fixed order and
// writes rs (visible after the caller's next barrier). Larger nt loops.
struct RmsRegs {
  float v[16];
};
__device__ __forceinline__ void rms_issue(RmsRegs& R, Rsrc ss, int ld, int nt, int q, int xp, int xo, int M, int m0,
                                          int tbase) {
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int m = m0 + row;
  const int xr = (min(m, M - 1) / q) * xp + min(m, M - 1) % q + xo;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int t = tbase + part + 4 * k;
    R.v[k] = (m < M && t < nt) ? ldf_c(ss, (u32)(t * ld + xr) * 4u) : 0.f;
  }
}
__device__ __forceinline__ void rms_finish(float* rs, Rsrc ss, RmsRegs& R, int ld, int nt, int q, int xp, int xo,
                                           int M, int m0, int d, float eps) {
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) acc += R.v[k];
  for (int tb = 64; tb < nt; tb += 64) {
    rms_issue(R, ss, ld, nt, q, xp, xo, M, m0, tb);
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += R.v[k];
  }
  acc += __shfl_xor(acc, 1, WAVE);
  acc += __shfl_xor(acc, 2, WAVE);
  const int row = threadIdx.x >> 2;
  if ((threadIdx.x & 3) == 0) rs[row] = m0 + row < M ? rsqrtf(acc / (float)d + eps) : 1.f;
}

// sum over the four lanes (g = 0..3) that share a tile row
__device__ __forceinline__ float sum_g(float v) {
  v += __shfl_xor(v, 16, WAVE);
  v += __shfl_xor(v, 32, WAVE);
  return v;
}

__device__ __forceinline__ void rope2(const float2* rope, int dh, int pos, int c, float& x0, float& x1) {
  const float2 cs = rope[(int64_t)pos * (dh >> 1) + (c >> 1)];
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

// ------------------------------------------------------------------ attention item
// One query (row `row`, head h) over positions lo..hi of a key/value store whose
// (sequence, head) block starts at kbase/vbase with slot(p) = ring ? (p-1) % cap : p-1.
// A group of DH/8 lanes owns one key at a time (16-byte loads); each group runs an
// online softmax over its keys, UNR keys per round with all K/V loads issued first;
// the groups are combined through LDS at the end.
template <int DH, int COH>
__device__ void attn_item(Rsrc qr, int row, int h, int hd, const bf16_t* kbase, const bf16_t* vbase, int ring,
                          int cap, int lo, int hi, float scale, Rsrc orr, float* lds) {
  constexpr int VEC = 8, G = DH / VEC, NG = kScanThreads / G, UNR = 8;
  constexpr int aux = COH ? SC1 : 0;
  const int tid = threadIdx.x, gi = tid / G, gl = tid % G;
  const int n = hi - lo + 1;
  float qv[VEC];
  unpack8(ld16c(qr, (u32)(row * hd + h * DH + gl * VEC) * 2u), qv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] *= scale;
  const Rsrc kr = mk(kbase), vr = mk(vbase);
  float m_run = -INFINITY, l_run = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int j0 = gi; j0 < n; j0 += NG * UNR) {
    u32x4 kk[UNR], vv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + u * NG;
      if (j < n) {
        const int p = lo + j;
        const int slot = ring ? (p - 1) % cap : p - 1;
        const u32 off = (u32)(slot * DH + gl * VEC) * 2u;
        kk[u] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, aux);
        vv[u] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, aux);
      }
    }
    float sc[UNR];
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float dot = -INFINITY;
      if (j0 + u * NG < n) {
        float kf[VEC];
        unpack8(kk[u], kf);
        dot = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) dot = fmaf(qv[e], kf[e], dot);
      }
#pragma unroll
      for (int o = G / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, WAVE);
      sc[u] = dot;
      mx = fmaxf(mx, dot);
    }
    const float corr = __expf(m_run - mx);
    l_run *= corr;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= corr;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (j0 + u * NG < n) {
        const float pw = __expf(sc[u] - mx);
        l_run += pw;
        float vf[VEC];
        unpack8(vv[u], vf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pw, vf[e], acc[e]);
      }
    }
    m_run = mx;
  }
  float* part = lds;                 // [NG][DH] partial numerators
  float* ml = lds + NG * DH;         // [NG][2] (max, denominator)
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[gi * DH + gl * VEC + e] = acc[e];
  if (gl == 0) { ml[2 * gi] = m_run; ml[2 * gi + 1] = l_run; }
  __syncthreads();
  if (tid < DH / 2) {
    float M = -INFINITY;
    for (int gg = 0; gg < NG; ++gg) M = fmaxf(M, ml[2 * gg]);
    float s0 = 0.f, s1 = 0.f, den = 0.f;
    for (int gg = 0; gg < NG; ++gg) {
      const float w = __expf(ml[2 * gg] - M);
      den += w * ml[2 * gg + 1];
      s0 += w * part[gg * DH + 2 * tid];
      s1 += w * part[gg * DH + 2 * tid + 1];
    }
    const float inv = 1.f / den;
    st4c(orr, (u32)(row * hd + h * DH + 2 * tid) * 2u, pack2(s0 * inv, s1 * inv));
  }
  __syncthreads();
}

// ------------------------------------------------------------------ row work
// z row <- src row (fp32), zb row <- bf16(src * gain), ssp[t][row] <- sum of squares of features 16t..16t+15
__device__ void row_entry(const float* src, Rsrc zr, Rsrc zbr, Rsrc ssr, int row, int ld_ss, const float* gain, int d,
                          bool write_z) {
  for (int c = threadIdx.x * 4; c < d; c += kScanThreads * 4) {
    const float4 v = *reinterpret_cast<const float4*>(src + c);
    if (write_z) {
      u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
      st16c(zr, (u32)(row * d + c) * 4u, w);
    }
    u32x2 b = {pack2(v.x * gain[c], v.y * gain[c + 1]), pack2(v.z * gain[c + 2], v.w * gain[c + 3])};
    st8c(zbr, (u32)(row * d + c) * 2u, b);
    float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    ss += __shfl_xor(ss, 1, WAVE);
    ss += __shfl_xor(ss, 2, WAVE);
    if ((threadIdx.x & 3) == 0) st4c(ssr, (u32)((c / 16) * ld_ss + row) * 4u, __float_as_uint(ss));
  }
}

// ------------------------------------------------------------------ kernel
constexpr int kMaxScanLayers = 64;

template <int DH, int OCC>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(OCC, 8)))
void scan_kernel(const ScanParams p) {
  extern __shared__ float smem[];
  __shared__ f32x4 red4[4][4][WAVE];
  __shared__ float rs[64];
  __shared__ int s_flag;
  __shared__ ScanLayer lay[kMaxScanLayers];
  u32 epoch = 0;
  const int d = p.d, hd = p.hd, H = p.H, B = p.B, f = p.f;
  const int P = p.P;                 // buffer rows per sequence: row of (b, i) is b * P + i
  const int ld_ss = B * P;
  {
    // the layer table is constant for the launch: keep it in LDS
    const uint64_t* src = reinterpret_cast<const uint64_t*>(p.layer);
    uint64_t* dst = reinterpret_cast<uint64_t*>(lay);
    const int nw = p.L * (int)(sizeof(ScanLayer) / 8);
    for (int i = threadIdx.x; i < nw; i += kScanThreads) dst[i] = src[i];
  }
  // scheduling group: the whole grid, or (ngroups = 8 * blocks per CU) the blocks of one
  // dispatch round on one XCD, owning B / ngroups sequences. Blocks are dealt to XCDs
  // round robin, so block i sits on XCD i % 8; its dispatch round is (i / 8) / (CUs per XCD).
  const int ngr = p.ngroups;
  int grp = 0, rank = blockIdx.x, nmem = gridDim.x;
  if (ngr > 1) {
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    grp = x + 8 * (k / p.cpx);
    rank = k % p.cpx;
    nmem = p.cpx;
  }
  const int Bg = B / ngr, b0g = grp * Bg;
  auto sync = [&]() -> bool {
    return ngr == 1 ? grid_sync(p.bar, epoch, &s_flag) : group_sync(p.bar, epoch, &s_flag, grp, rank, nmem);
  };
  const int ntn_m = 2 * d / 16, ntm_m = (Bg + 63) / 64;   // merge GEMM tiles
  WPre wpre;
  // weights of this block's first tile of a GEMM phase with N rows, K columns and ntm row tiles
  auto prefetch = [&](const bf16_t* W, int N, int K, int ntm_) {
    const int ntn = N / 16;
    if (rank < ntn * ntm_) w_prefetch(wpre, W, N, K, (rank % ntn) * 16);
  };

  // PROLOGUE: register rows in the consumed form (bf16(rho * ns), sums of squares)
  if (p.variant != V0_) {
    const Rsrc rhob_r = mk(p.rhob), rhoss_r = mk(p.rhoss);
    for (int b = b0g + rank; b < b0g + Bg; b += nmem)
      row_entry(p.rho + (int64_t)b * d, rhob_r, rhob_r, rhoss_r, b, B, p.ns, d, false);
    if (p.T > 0) prefetch(p.wsr, 2 * d, d, ntm_m);
  }
  if (!sync()) return;

  int t0 = p.start;
  const int end = p.start + p.T;
  int pass = 0, np_prev = 0;
  bool prev_complete = false;
  const int nt_last = p.L > 0 ? d / 16 : d / 8;   // sum-of-squares tiles of a pass's final output
  while (true) {
    const bool have = t0 < end;
    int np = 0;
    if (have) {
      if (p.variant == V2_) np = min(end, (t0 / p.chunk + 1) * p.chunk) - t0;
      else if (p.variant == V0_) np = min(end - t0, P);
      else np = 1;
    }
    const int par = pass & 1, ppar = par ^ 1;
    const int r0 = b0g * np, r1 = (b0g + Bg) * np;      // this group's rows (compact index b * np + i)
    const int grows = r1 - r0;
    const int ntm = (grows + 63) / 64;

    // ---------------- MERGE / INIT phase (+ finishing rows of the previous pass)
    {
      const Rsrc z_r = mk(p.z[par]), zb_r = mk(p.zb[par]), ss_r = mk(p.ssp[par]);
      const Rsrc pz_r = mk(p.z[ppar]);
      int nwork = 0;
      if (have) nwork = p.variant == V0_ ? grows : ntn_m * ntm_m;
      const int nfin = Bg * np_prev;
      for (int it = rank; it < nwork + nfin; it += nmem) {
        if (it < nwork) {
          if (p.variant == V0_) {
            const int cm = r0 + it;
            const int b = cm / np, i = cm % np;
            row_entry(p.e + ((int64_t)b * p.Tm + t0 + i) * d, z_r, zb_r, ss_r, b * P + i, ld_ss, p.g_first, d, true);
          } else {
            const int tn = it % ntn_m, tm = it / ntn_m;
            const int n0 = tn * 16, m0 = b0g + tm * 64, Mend = b0g + Bg;
            const int nmb = min(4, (Mend - m0 + 15) / 16);
            // merge input: last rows of the previous pass when it closed a chunk, else the register
            const bool from_prev = pass > 0 && prev_complete;
            const Rsrc xr = mk(from_prev ? (const void*)p.zb[ppar] : (const void*)p.rhob);
            const Rsrc ssrc = mk(from_prev ? (const void*)p.ssp[ppar] : (const void*)p.rhoss);
            const int xp = from_prev ? P : 1, xo = from_prev ? np_prev - 1 : 0;
            const int ssld = from_prev ? ld_ss : B, ssnt = from_prev ? nt_last : d / 16;
            RmsRegs R;
            rms_issue(R, ssrc, ssld, ssnt, 1, xp, xo, Mend, m0, 0);
            tile_mma(p.wsr, 2 * d, d, n0, xr, d, 1, xp, xo, Mend, m0, nmb, red4, it == rank ? &wpre : nullptr);
            rms_finish(rs, ssrc, R, ssld, ssnt, 1, xp, xo, Mend, m0, d, p.eps);
            __syncthreads();
            const f32x4 acc = tile_sum(nmb, red4);
            const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
            const int b = m0 + wave * 16 + (lane & 15);
            const int n = n0 + 4 * (lane >> 4);
            const bool valid = wave < nmb && b < Mend;
            const float r = valid ? rs[wave * 16 + (lane & 15)] : 0.f;
            const float ga = acc[0] * r, sa = acc[1] * r, gb = acc[2] * r, sb = acc[3] * r;
            const int j = n >> 1;
            for (int rep = 0; rep < np; ++rep) {
              float u0 = 0.f, u1 = 0.f;
              const int row = b * P + rep;
              if (valid) {
                const int64_t eo = ((int64_t)b * p.Tm + t0 + rep) * d + j;
                u0 = p.e[eo] + p.alpha * sigmoidf_(p.gpre[eo] + ga) * sa;
                u1 = p.e[eo + 1] + p.alpha * sigmoidf_(p.gpre[eo + 1] + gb) * sb;
                st8c(z_r, (u32)(row * d + j) * 4u, u32x2{__float_as_uint(u0), __float_as_uint(u1)});
                st4c(zb_r, (u32)(row * d + j) * 2u, pack2(u0 * p.g_first[j], u1 * p.g_first[j + 1]));
              }
              const float ss = sum_g(u0 * u0 + u1 * u1);
              if (valid && (lane >> 4) == 0) st4c(ss_r, (u32)(tn * ld_ss + row) * 4u, __float_as_uint(ss));
            }
          }
        } else {
          // finish the previous pass: s_t of every position, s and the register of the last position
          const int cm = b0g * np_prev + (it - nwork);
          const int b = cm / np_prev, i = cm % np_prev;
          const int row = b * P + i;
          const int tp = t0 - np_prev + i;          // 0-based position index of this row
          const bool last = i == np_prev - 1;
          const bool reg = last && prev_complete && p.variant != V0_;
          const Rsrc pzb_r = mk(p.zb[ppar]), pss_r = mk(p.ssp[ppar]);
          const Rsrc rhob_r = mk(p.rhob), rhoss_r = mk(p.rhoss);
          for (int c = threadIdx.x * 4; c < d; c += kScanThreads * 4) {
            const u32x4 v = ld16c(pz_r, (u32)(row * d + c) * 4u);
            const float4 fv = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                                          __uint_as_float(v[3]));
            *reinterpret_cast<float4*>(p.sall + ((int64_t)b * p.Tm + tp) * d + c) = fv;
            if (last) *reinterpret_cast<float4*>(p.s + (int64_t)b * d + c) = fv;
            if (reg) {
              *reinterpret_cast<float4*>(p.rho + (int64_t)b * d + c) = fv;
              const u32x2 zb4 = __builtin_amdgcn_raw_buffer_load_b64(pzb_r, (u32)(row * d + c) * 2u, 0, SC1);
              st8c(rhob_r, (u32)(b * d + c) * 2u, zb4);
            }
          }
          if (reg) {
            for (int t = threadIdx.x; t < d / 16; t += kScanThreads) {
              float v = 0.f;
              if (nt_last == d / 16) v = ldf_c(pss_r, (u32)(t * ld_ss + row) * 4u);
              else v = ldf_c(pss_r, (u32)(2 * t * ld_ss + row) * 4u) + ldf_c(pss_r, (u32)((2 * t + 1) * ld_ss + row) * 4u);
              st4c(rhoss_r, (u32)(t * B + b) * 4u, __float_as_uint(v));
            }
          }
        }
        __syncthreads();
      }
    }
    if (!have) break;
    if (p.L > 0) prefetch(lay[0].wqkv, 3 * hd, d, ntm);
    else if (t0 + np < end) prefetch(p.wsr, 2 * d, d, ntm_m);
    if (!sync()) return;

    // ---------------- decoder layers
    const Rsrc z_r = mk(p.z[par]), zb_r = mk(p.zb[par]), ss_r = mk(p.ssp[par]);
    const Rsrc q_r = mk(p.q), ao_r = mk(p.ao), hid_r = mk(p.hid);
    int nt_in = p.variant == V0_ ? d / 16 : d / 8;   // merge output: 8 features per tile
    for (int l = 0; l < p.L; ++l) {
      const ScanLayer& Ly = lay[l];
      // QKV: q (RoPE) -> q, k (RoPE) and v -> ring slot (pos - 1) % R
      {
        const Rsrc rk_r = mk(Ly.rk), rv_r = mk(Ly.rv);
        const int N = 3 * hd, ntn = N / 16;
        for (int it = rank; it < ntn * ntm; it += nmem) {
          const int tn = it % ntn, tm = it / ntn;
          const int n0 = tn * 16, m0 = r0 + tm * 64, nmb = min(4, (r1 - m0 + 15) / 16);
          RmsRegs R;
          rms_issue(R, ss_r, ld_ss, nt_in, np, P, 0, r1, m0, 0);
          tile_mma(Ly.wqkv, N, d, n0, zb_r, d, np, P, 0, r1, m0, nmb, red4, it == rank ? &wpre : nullptr);
          rms_finish(rs, ss_r, R, ld_ss, nt_in, np, P, 0, r1, m0, d, p.eps);
          __syncthreads();
          const f32x4 acc = tile_sum(nmb, red4);
          const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
          const int cm = m0 + wave * 16 + (lane & 15), n = n0 + 4 * (lane >> 4);
          if (wave < nmb && cm < r1) {
            const float r = rs[wave * 16 + (lane & 15)];
            float v0 = acc[0] * r, v1 = acc[1] * r, v2 = acc[2] * r, v3 = acc[3] * r;
            const int b = cm / np, i = cm % np, pos = t0 + 1 + i, m = b * P + i;
            const int region = n / hd, w = n - region * hd, h = w / DH, c = w % DH;
            if (region < 2) {
              rope2(p.rope, DH, pos, c, v0, v1);
              rope2(p.rope, DH, pos, c + 2, v2, v3);
            }
            const u32x2 pk = {pack2(v0, v1), pack2(v2, v3)};
            if (region == 0) {
              st8c(q_r, (u32)(m * hd + w) * 2u, pk);
            } else {
              const int slot = (pos - 1) % p.R;
              const u32 off = (u32)((((int64_t)b * H + h) * p.R + slot) * DH + c) * 2u;
              if (region == 1) st8c(rk_r, off, pk);
              else st8c(rv_r, off, pk);
            }
          }
          __syncthreads();
        }
      }
      if (!sync()) return;
      // SWA over the ring: keys max(1, pos - W + 1) .. pos
      for (int it = rank; it < grows * H; it += nmem) {
        const int cm = r0 + it / H, h = it % H;
        const int b = cm / np, i = cm % np, pos = t0 + 1 + i, m = b * P + i;
        const int64_t hb = (((int64_t)b * H + h) * p.R) * DH;
        attn_item<DH, 1>(q_r, m, h, hd, Ly.rk + hb, Ly.rv + hb, 1, p.R, max(1, pos - p.W + 1), pos, p.scale, ao_r,
                         smem);
      }
      prefetch(Ly.wo, d, hd, ntm);
      if (!sync()) return;
      // residual GEMM: z += W x (x = attention output or SwiGLU hidden); zb = bf16(z * gnext); ssp
      auto residual = [&](const bf16_t* Wm, int K, const bf16_t* xptr, const float* gnext) {
        const int N = d, ntn = N / 16;
        const Rsrc xr = mk(xptr);
        for (int it = rank; it < ntn * ntm; it += nmem) {
          const int tn = it % ntn, tm = it / ntn;
          const int n0 = tn * 16, m0 = r0 + tm * 64, nmb = min(4, (r1 - m0 + 15) / 16);
          const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
          const int cm = m0 + wave * 16 + (lane & 15), n = n0 + 4 * (lane >> 4);
          const bool valid = wave < nmb && cm < r1;
          const int m = (cm / np) * P + cm % np;
          u32x4 o = {0u, 0u, 0u, 0u};
          if (valid) o = ld16c(z_r, (u32)(m * d + n) * 4u);     // residual operand, loaded with the tile
          tile_mma(Wm, N, K, n0, xr, K, np, P, 0, r1, m0, nmb, red4, it == rank ? &wpre : nullptr);
          __syncthreads();
          const f32x4 acc = tile_sum(nmb, red4);
          float ss = 0.f;
          if (valid) {
            const float z0 = __uint_as_float(o[0]) + acc[0], z1 = __uint_as_float(o[1]) + acc[1];
            const float z2 = __uint_as_float(o[2]) + acc[2], z3 = __uint_as_float(o[3]) + acc[3];
            st16c(z_r, (u32)(m * d + n) * 4u,
                  u32x4{__float_as_uint(z0), __float_as_uint(z1), __float_as_uint(z2), __float_as_uint(z3)});
            st8c(zb_r, (u32)(m * d + n) * 2u,
                 u32x2{pack2(z0 * gnext[n], z1 * gnext[n + 1]), pack2(z2 * gnext[n + 2], z3 * gnext[n + 3])});
            ss = z0 * z0 + z1 * z1 + z2 * z2 + z3 * z3;
          }
          ss = sum_g(ss);
          if (valid && (lane >> 4) == 0) st4c(ss_r, (u32)(tn * ld_ss + m) * 4u, __float_as_uint(ss));
          __syncthreads();
        }
      };
      residual(Ly.wo, hd, p.ao, Ly.g2);
      nt_in = d / 16;
      prefetch(Ly.xq, hd, d, ntm);
      if (!sync()) return;
      // cross-attention query: Xq (RoPE at pos)
      {
        const int N = hd, ntn = N / 16;
        for (int it = rank; it < ntn * ntm; it += nmem) {
          const int tn = it % ntn, tm = it / ntn;
          const int n0 = tn * 16, m0 = r0 + tm * 64, nmb = min(4, (r1 - m0 + 15) / 16);
          RmsRegs R;
          rms_issue(R, ss_r, ld_ss, nt_in, np, P, 0, r1, m0, 0);
          tile_mma(Ly.xq, N, d, n0, zb_r, d, np, P, 0, r1, m0, nmb, red4, it == rank ? &wpre : nullptr);
          rms_finish(rs, ss_r, R, ld_ss, nt_in, np, P, 0, r1, m0, d, p.eps);
          __syncthreads();
          const f32x4 acc = tile_sum(nmb, red4);
          const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
          const int cm = m0 + wave * 16 + (lane & 15), n = n0 + 4 * (lane >> 4);
          if (wave < nmb && cm < r1) {
            const float r = rs[wave * 16 + (lane & 15)];
            float v0 = acc[0] * r, v1 = acc[1] * r, v2 = acc[2] * r, v3 = acc[3] * r;
            const int pos = t0 + 1 + cm % np, c = n % DH, m = (cm / np) * P + cm % np;
            rope2(p.rope, DH, pos, c, v0, v1);
            rope2(p.rope, DH, pos, c + 2, v2, v3);
            st8c(q_r, (u32)(m * hd + n) * 2u, u32x2{pack2(v0, v1), pack2(v2, v3)});
          }
          __syncthreads();
        }
      }
      if (!sync()) return;
      // CROSS over the memory prefix 1..pos of this layer's group
      for (int it = rank; it < grows * H; it += nmem) {
        const int cm = r0 + it / H, h = it % H;
        const int b = cm / np, pos = t0 + 1 + cm % np, m = b * P + cm % np;
        const int64_t hb = (((int64_t)b * H + h) * p.Tm) * DH;
        attn_item<DH, 0>(q_r, m, h, hd, Ly.mk + hb, Ly.mv + hb, 0, p.Tm, 1, pos, p.scale, ao_r, smem);
      }
      prefetch(Ly.xo, d, hd, ntm);
      if (!sync()) return;
      residual(Ly.xo, hd, p.ao, Ly.g3);
      prefetch(Ly.w13, 2 * f, d, ntm);
      if (!sync()) return;
      // W13 + SwiGLU -> hid
      {
        const int N = 2 * f, ntn = N / 16;
        for (int it = rank; it < ntn * ntm; it += nmem) {
          const int tn = it % ntn, tm = it / ntn;
          const int n0 = tn * 16, m0 = r0 + tm * 64, nmb = min(4, (r1 - m0 + 15) / 16);
          RmsRegs R;
          rms_issue(R, ss_r, ld_ss, nt_in, np, P, 0, r1, m0, 0);
          tile_mma(Ly.w13, N, d, n0, zb_r, d, np, P, 0, r1, m0, nmb, red4, it == rank ? &wpre : nullptr);
          rms_finish(rs, ss_r, R, ld_ss, nt_in, np, P, 0, r1, m0, d, p.eps);
          __syncthreads();
          const f32x4 acc = tile_sum(nmb, red4);
          const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
          const int cm = m0 + wave * 16 + (lane & 15), n = n0 + 4 * (lane >> 4);
          if (wave < nmb && cm < r1) {
            const float r = rs[wave * 16 + (lane & 15)];
            const int m = (cm / np) * P + cm % np;
            const float a0 = acc[0] * r, b0 = acc[1] * r, a1 = acc[2] * r, b1 = acc[3] * r;
            st4c(hid_r, (u32)(m * f + (n >> 1)) * 2u, pack2(a0 * sigmoidf_(a0) * b0, a1 * sigmoidf_(a1) * b1));
          }
          __syncthreads();
        }
      }
      prefetch(Ly.w2, d, f, ntm);
      if (!sync()) return;
      residual(Ly.w2, f, p.hid, Ly.gnext);
      if (l + 1 < p.L) prefetch(lay[l + 1].wqkv, 3 * hd, d, ntm);
      else if (p.variant != V0_ && t0 + np < end) prefetch(p.wsr, 2 * d, d, ntm_m);
      if (!sync()) return;
    }
    if (p.L == 0 && !sync()) return;
    prev_complete = p.variant == V0_ ? false : (p.variant != V2_ || (t0 + np) % p.chunk == 0);
    np_prev = np;
    t0 += np;
    pass += 1;
  }
}

bool scan_supported(int dh, int rows, int d, int hd, int f, int Tm, int L) {
  return (dh == 64 || dh == 128) && L <= kMaxScanLayers && rows <= 4096 && d % 64 == 0 && hd % 64 == 0 && f % 64 == 0 &&
         (int64_t)rows * (f > d ? f : d) * 4 < (1ll << 31);
}

int scan_lds_bytes(int Tm, int W, int R, int dh) {
  const int ng = kScanThreads / (dh / 8);
  return 4 * (ng * dh + 2 * ng);
}

int scan_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

hipError_t launch_scan(const ScanParams& p, int* grid_out, hipStream_t st) {
  const int cus = scan_cus();
  if (cus < 8 || cus % 8) return hipErrorInvalidConfiguration;
  const int bpc = p.ngroups == 1 ? 1 : p.ngroups / 8;
  const int lds = scan_lds_bytes(p.Tm, p.W, p.R, p.dh);
  const void* fn = nullptr;
  if (p.dh == 64) fn = bpc >= 4 ? (const void*)scan_kernel<64, 4> : bpc == 2 ? (const void*)scan_kernel<64, 2> : (const void*)scan_kernel<64, 1>;
  else fn = bpc >= 4 ? (const void*)scan_kernel<128, 4> : bpc == 2 ? (const void*)scan_kernel<128, 2> : (const void*)scan_kernel<128, 1>;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kScanThreads, lds);
  if (e != hipSuccess) return e;
  if (occ < bpc || p.cpx * 8 != cus) return hipErrorInvalidConfiguration;
  const int grid = cus * bpc;
  *grid_out = grid;
  ScanParams arg = p;
  void* args[] = {&arg};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kScanThreads), args, lds, st);
}

}  // namespace rlt
