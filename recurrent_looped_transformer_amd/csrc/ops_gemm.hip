// GEMM kernels with fused epilogues.
//
// Y[m, n] = sum_k X[m, k] W[n, k] with W the packed weight [N, K] (K contiguous)
// and X activations [M, K]. The weight is the MFMA "A" operand, so each lane of a
// 16x16 output tile holds four consecutive output features n..n+3 of one row m:
// row pairs packed next to each other (rotary pairs, SwiGLU W1/W3 rows, merge
// gate/state rows) meet in one lane and the epilogue needs no shuffles.
//
//  - gemm_skinny: decode shapes (M = batch rows <= a few hundred). One
//    workgroup streams 16 weight rows once for up to 64 activation rows; eight
//    waves split K, keep the tile's loads in flight together and reduce through
//    LDS. Bandwidth-bound on the weights. Carries the folded RMSNorm (see EpArgs).
//  - gemm_large: prefill shapes, 256x256 tiles (see below).
//  - gemm_tiled: prefill fallback. 128x128 tiles, K step 32, LDS double
//    buffer, 4 waves x (64x64) of 16x16x32 MFMAs.
//  The 16-bit kernels take T = bf16_t or f16_t (storage and MFMA input type).
//  - gemm_f32: the fp32 configuration (vector FMA).
#include <stdio.h>
#include <stdlib.h>

#include "common.hpp"
#include "ops.hpp"

namespace rlt {

__device__ __forceinline__ float2 rope_cs(const EpArgs& a, int pos, int c) {
  return a.rope[(int64_t)pos * (a.dh >> 1) + (c >> 1)];
}
__device__ __forceinline__ void rope_apply(float2 cs, float& x0, float& x1) {
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

// Position index (0-based) before the first position of row m's sequence in this call.
// (a.pos0 passes through readfirstlane, an identity on this uniform value: otherwise the
// compiler merges the three loads into one load from a chosen address, and the argument's
// address space forces a copy of it to per-lane scratch memory and a flat load)
__device__ __forceinline__ int ep_pos0(const EpArgs& a, int m) {
  int p = __builtin_amdgcn_readfirstlane(a.pos0);
  if (a.row_pos) p = a.row_pos[m / a.tn];
  else if (a.pos_dev) p = a.pos_dev[0];
  return p;
}

// Epilogue operands a decode GEMM loads before its main loop (they do not depend on it):
// the residual row and the next norm's gain, or the rotary factors of the lane's features.
struct EpPre {
  float4 z, g;
  float2 cs0, cs1;
};
template <Ep E, bool kFold>
__device__ __forceinline__ EpPre ep_prefetch(const EpArgs& a, int m, int n) {
  EpPre p{};
  if constexpr (E == Ep::Residual) {
    p.z = *reinterpret_cast<const float4*>(a.resid + a.rmap.off(m) + n);
    if (kFold && a.fold_zb) p.g = *reinterpret_cast<const float4*>(a.fold_gain + n);
  } else if constexpr (E == Ep::RopeQ || E == Ep::QKV || E == Ep::MemKV) {
    // same position and channel as the epilogue below (rows m = b * tn + i, position pos0 + 1 + i)
    const int pos = ep_pos0(a, m) + 1 + (m % a.tn);
    const int c = E == Ep::RopeQ ? n % a.dh : (n % a.hd) % a.dh;
    p.cs0 = rope_cs(a, pos, c);
    p.cs1 = rope_cs(a, pos, c + 2);
  }
  return p;
}

// kv slot address (elements) of (sequence b, head h, position pos, channel c)
__device__ __forceinline__ int64_t kv_off(const EpArgs& a, int b, int h, int pos, int c) {
  const int slot = a.kv.ring ? (pos - 1) % a.kv.cap : pos - 1;
  return (((int64_t)(a.b0 + b) * a.H + h) * a.kv.cap + slot) * a.dh + c;
}

// Applies the epilogue to acc values v of row m, features n..n+3. Returns the sum of
// squares of the new residual values when the Residual epilogue folds the next RMSNorm
// (fold_zb set), else 0.
template <typename T, Ep E, bool kFold = false>
__device__ __forceinline__ float epilogue(const EpArgs& a, int m, int n, float v[4], const EpPre* pre = nullptr) {
  T* out = reinterpret_cast<T*>(a.out);
  if constexpr (E == Ep::StoreAct) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Elem<T>::st(out + (int64_t)m * a.ldo + n + i, v[i]);
  } else if constexpr (E == Ep::StoreF32) {
    float* o = reinterpret_cast<float*>(a.out) + (int64_t)m * a.ldo + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = v[i];
  } else if constexpr (E == Ep::Residual) {
    float* r = a.resid + a.rmap.off(m) + n;
    // both loads before any store: the stores may alias the gain as far as the compiler knows
    const float4 old = pre ? pre->z : *reinterpret_cast<const float4*>(r);
    const float4 gn = !(kFold && a.fold_zb) ? make_float4(0.f, 0.f, 0.f, 0.f)
                      : pre ? pre->g : *reinterpret_cast<const float4*>(a.fold_gain + n);
    const float z[4] = {old.x + v[0], old.y + v[1], old.z + v[2], old.w + v[3]};
    const float4 z4 = make_float4(z[0], z[1], z[2], z[3]);
    *reinterpret_cast<float4*>(r) = z4;
    if (a.dup_rows) *reinterpret_cast<float4*>(a.dup_rows + a.dup_map.off(m) + n) = z4;
    if (a.dup_last && m % a.tn == a.tn - 1)
      *reinterpret_cast<float4*>(a.dup_last + (int64_t)(m / a.tn) * a.dup_last_ld + n) = z4;
    if (kFold && a.fold_zb) {
      T* zb = reinterpret_cast<T*>(a.fold_zb) + (int64_t)m * a.fold_ld + n;
      store_act<T>(zb, a.out_split, z[0] * gn.x);
      store_act<T>(zb + 1, a.out_split, z[1] * gn.y);
      store_act<T>(zb + 2, a.out_split, z[2] * gn.z);
      store_act<T>(zb + 3, a.out_split, z[3] * gn.w);
      return z[0] * z[0] + z[1] * z[1] + z[2] * z[2] + z[3] * z[3];
    }
  } else if constexpr (E == Ep::Bias) {
    float* r = a.resid + a.rmap.off(m) + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = v[i] + a.bias[n + i];
  } else if constexpr (E == Ep::SwiGLU) {
    T* o = out + (int64_t)m * a.ldo + (n >> 1);
    store_act<T>(o, a.out_split, v[0] * sigmoidf_(v[0]) * v[1]);
    store_act<T>(o + 1, a.out_split, v[2] * sigmoidf_(v[2]) * v[3]);
  } else if constexpr (E == Ep::RopeQ) {
    const int pos = ep_pos0(a, m) + 1 + (m % a.tn);
    const int c = n % a.dh;
    rope_apply(pre ? pre->cs0 : rope_cs(a, pos, c), v[0], v[1]);
    rope_apply(pre ? pre->cs1 : rope_cs(a, pos, c + 2), v[2], v[3]);
    T* o = out + (int64_t)m * a.ldo + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) Elem<T>::st(o + i, v[i]);
  } else if constexpr (E == Ep::QKV || E == Ep::MemKV) {
    const int b = m / a.tn, i = m % a.tn;
    const int pos = ep_pos0(a, m) + 1 + i;
    int region = n / a.hd;
    const int w = n - region * a.hd;
    if constexpr (E == Ep::MemKV) region += 1;   // memory projection has no query part
    const int h = w / a.dh, c = w % a.dh;
    if (region < 2) {
      rope_apply(pre ? pre->cs0 : rope_cs(a, pos, c), v[0], v[1]);
      rope_apply(pre ? pre->cs1 : rope_cs(a, pos, c + 2), v[2], v[3]);
    }
    T* dst;
    int64_t lo;
    if (region == 0) {
      dst = out + (int64_t)m * a.ldo + w;
      lo = a.out_split;
    } else {
      dst = reinterpret_cast<T*>(region == 1 ? a.kv.k : a.kv.v) + kv_off(a, b, h, pos, c);
      lo = a.kv.lo;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) store_act<T>(dst + k, lo, v[k]);
  } else if constexpr (E == Ep::Merge) {
    // rows (2j, 2j+1) of the packed [W_g,r ; W_s] weight: gate part and state projection of feature j
    const int j = n >> 1;
    const int64_t e0 = a.row_pos ? (int64_t)a.row_pos[m] * a.pos_stride
                     : a.pos_dev ? (int64_t)a.pos_dev[0] * a.pos_stride : 0;
    float u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int rep = 0; rep < a.nrep; ++rep) {
      const int64_t eo = e0 + (int64_t)m * a.eb + (int64_t)rep * a.et + j;
      float* z = a.resid + a.rmap.off(m * a.nrep + rep) + j;
      u0 = a.e[eo] + a.alpha * sigmoidf_(a.gpre[eo] + v[0]) * v[1];
      u1 = a.e[eo + 1] + a.alpha * sigmoidf_(a.gpre[eo + 1] + v[2]) * v[3];
      z[0] = u0;
      z[1] = u1;
    }
    if (kFold && a.fold_zb) {   // nrep == 1: u0, u1 are this row's features j, j + 1
      T* zb = reinterpret_cast<T*>(a.fold_zb) + (int64_t)m * a.fold_ld + j;
      store_act<T>(zb, a.out_split, u0 * a.fold_gain[j]);
      store_act<T>(zb + 1, a.out_split, u1 * a.fold_gain[j + 1]);
      return u0 * u0 + u1 * u1;
    }
  }
  return 0.f;
}

// ------------------------------------------------------------------ skinny (decode)
// One workgroup of kSkW waves owns TPW tiles of 16 output features and 16 * NMB rows. The
// waves split K into 64-wide chunks (chunk c to wave c % kSkW) and each wave issues the
// weight and activation loads of U chunks before their MFMAs, so that the workgroup's whole
// weight slice is in flight at once for K up to kSkW * U * 64; every activation fragment a
// wave loads feeds the TPW weight tiles (fewer re-reads of X when N is large). Partial tiles
// meet in LDS. A row's sums run in the same order for every TPW, NMB and M.
//
// K split (gridDim.z = S > 1): workgroup z takes the z-th run of K / 64 / S chunks and stores
// its reduced tiles, unscaled, to the split-K workspace; skinny_reduce then adds the S partial
// tiles of every output tile in split order 0 .. S-1 and runs the row scale and epilogue.
// With many rows every workgroup reads all of them for its K range, so cutting K cuts the
// activation bytes each workgroup reads per weight byte (at 64 two-term rows, 128 activation
// rows per weight tile). (One kernel whose last-arriving workgroup finished the tiles, after
// a device-scope release of its partials, measured 3x slower at the paper shape: each
// release writes back the L2 of its XCD.)
constexpr int kSkW = 8;

template <int TPW, int NMB>
constexpr int skinny_unroll() {
  return TPW + NMB <= 2 ? 8 : (TPW + NMB <= 4 ? 4 : (TPW + NMB <= 6 ? 2 : 1));
}

// Row scales of the folded RMSNorm (consumer side) of rows m0 .. m0 + 16 NMB - 1 into rsl:
// wave w reduces rows w, w + kSkW, ... from the float4 partial sums ssr it loaded.
template <int NMB>
__device__ __forceinline__ void skinny_scales(const EpArgs& a, const float4* ssr, float* rsl, int wave, int lane) {
  constexpr int RPW = NMB * 16 / kSkW;
  const float live = lane * 4 < a.rs_n ? 1.f : 0.f;
  float tt[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) tt[i] = wave_sum_dpp((ssr[i].x + ssr[i].y + ssr[i].z + ssr[i].w) * live);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) rsl[wave + kSkW * i] = rsqrtf(tt[i] / (float)a.rs_d + a.rs_eps);
  }
}
template <int NMB>
__device__ __forceinline__ void skinny_scale_loads(const EpArgs& a, float4* ssr, int m0, int M, int wave, int lane) {
  constexpr int RPW = NMB * 16 / kSkW;
  const int k4 = min(lane * 4, a.rs_n - 4);
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int m = min(m0 + wave + kSkW * i, M - 1);
    ssr[i] = *reinterpret_cast<const float4*>(a.rs_ssp + (int64_t)m * a.rs_n + k4);
  }
}

// Epilogue of output tile o = t * NMB + j of a skinny workgroup (tiles tile0.., rows m0..):
// lane (r, g) holds rows m0 + 16 j + r, features (tile0 + t) * 16 + 4 g .. + 3.
template <typename T, Ep E, int NMB>
__device__ __forceinline__ void skinny_finish(const EpArgs& a, int M, int N, int tile0, int m0, int r, int g,
                                              const float* rsl, int o, f32x4 sum, const EpPre* pp) {
  const int t = o / NMB, j = o % NMB;
  const int m = m0 + j * 16 + r;
  const int n = (tile0 + t) * 16 + 4 * g;
  const float sc = a.rs_ssp ? rsl[j * 16 + r] : 1.f;
  float ss = 0.f;
  if (m < M && n < N) {
    float v[4] = {sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc};
    ss = epilogue<T, E, true>(a, m, n, v, pp);
  }
  if constexpr (E == Ep::Residual || E == Ep::Merge) {
    if (a.fold_zb) {
      // lanes r, r+16, r+32, r+48 hold the tile's features of row m (16, or 8 for Merge)
      ss += __shfl_xor(ss, 16, WAVE);
      ss += __shfl_xor(ss, 32, WAVE);
      if (g == 0 && m < M) a.fold_ssp[(int64_t)m * (N / 16) + tile0 + t] = ss;
    }
  }
}

// XS: two-term X (each row K hi terms, then K lo terms): every weight chunk loaded once feeds
// the MFMAs of both terms. NT: weight loads with the nontemporal hint (launches of one row
// block whose weights stream once per step from a set larger than the last-level cache).
// KS: a K-split launch (its own instances: the unsplit ones keep compile-time chunk bounds,
// measured 10% faster at one row than with the split bounds read from the grid).
template <typename T, Ep E, int NMB, int TPW, bool XS, bool NT = false, bool KS = false>
__global__ __launch_bounds__(kSkW * WAVE) void gemm_skinny(const T* __restrict__ X, int64_t ldx,
                                                           const T* __restrict__ W, int M, int N, int K,
                                                           EpArgs a) {
  constexpr int U = XS ? (skinny_unroll<TPW, NMB>() > 1 ? skinny_unroll<TPW, NMB>() / 2 : 1)
                       : skinny_unroll<TPW, NMB>();
  constexpr int NO = TPW * NMB;            // output tiles of the workgroup
  constexpr int NOB = NO < 4 ? NO : 4;     // output tiles reduced per pass (LDS: 32 KB)
  constexpr int RPW = NMB * 16 / kSkW;     // rows per wave in the row-scale prologue
  __shared__ f32x4 red[kSkW][NOB][WAVE];
  __shared__ float rsl[NMB * 16];
  const int tile0 = blockIdx.x * TPW;
  const int m0 = blockIdx.y * (NMB * 16);
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r = lane & 15, g = lane >> 4;

  // folded RMSNorm of the input rows: fetch the partial sums now (one float4 per lane and
  // row, no branches: rs_n is a multiple of 4), reduce after the main loop
  // (the loaded values stay untouched until then, so no wait is placed before the weight loads)
  // (a split launch stores unscaled partial tiles: the scales belong to skinny_reduce)
  const int ks = KS ? gridDim.z : 1;
  float4 ssr[RPW];
  if (a.rs_ssp && ks == 1) skinny_scale_loads<NMB>(a, ssr, m0, M, wave, lane);

  // the epilogue waves' operands (residual row, gain, rotary factors) are requested first;
  // in reduction pass p, wave w < NOB finishes output tile o = p NOB + w, (t, j) = (o / NMB,
  // o % NMB); the first pass's operands are prefetched
  EpPre pre{};
  if (wave < NOB && ks == 1) {
    const int em = m0 + (wave % NMB) * 16 + r, en = (tile0 + wave / NMB) * 16 + 4 * g;
    if (em < M && en < N) pre = ep_prefetch<E, true>(a, em, en);
  }
  const T* wp = W + (int64_t)tile0 * 16 * K + lane * 8;   // tile-major weight tiles
  const T* xp[NMB];
#pragma unroll
  for (int j = 0; j < NMB; ++j) xp[j] = X + (int64_t)min(m0 + j * 16 + r, M - 1) * ldx + g * 16;
  f32x4 acc[TPW][NMB];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < NMB; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two-term X: the lo terms of chunk c lie at chunk c + nch of the row
  const int nch = K / 64;
  const int cpk = KS ? nch / ks : nch;            // chunks per K split
  const int cb = KS ? blockIdx.z * cpk : 0, ce = KS ? cb + cpk : nch;
  for (int c0 = cb + wave; c0 < ce; c0 += kSkW * U) {
    uint4 wa[U][TPW][2], xb[U][NMB][2], xl[XS ? U : 1][NMB][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kSkW;
      if (c < ce) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          wa[u][t][0] = ld16<NT>(wp + (int64_t)t * 16 * K + c * 1024);
          wa[u][t][1] = ld16<NT>(wp + (int64_t)t * 16 * K + c * 1024 + 512);
        }
#pragma unroll
        for (int j = 0; j < NMB; ++j) {
          xb[u][j][0] = *reinterpret_cast<const uint4*>(xp[j] + c * 64);
          xb[u][j][1] = *reinterpret_cast<const uint4*>(xp[j] + c * 64 + 8);
          if constexpr (XS) {
            xl[u][j][0] = *reinterpret_cast<const uint4*>(xp[j] + (c + nch) * 64);
            xl[u][j][1] = *reinterpret_cast<const uint4*>(xp[j] + (c + nch) * 64 + 8);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * kSkW < ce) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int j = 0; j < NMB; ++j) {
            if constexpr (XS) {
              acc[t][j] = mfma16x16x32<T>(wa[u][t][0], xl[u][j][0], acc[t][j]);
              acc[t][j] = mfma16x16x32<T>(wa[u][t][1], xl[u][j][1], acc[t][j]);
            }
            acc[t][j] = mfma16x16x32<T>(wa[u][t][0], xb[u][j][0], acc[t][j]);
            acc[t][j] = mfma16x16x32<T>(wa[u][t][1], xb[u][j][1], acc[t][j]);
          }
      }
    }
  }
  if (a.rs_ssp && ks == 1) skinny_scales<NMB>(a, ssr, rsl, wave, lane);
  // partial tile o of split z of this workgroup's (row block, tile group), one f32x4 per lane
  const int64_t grp = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t zstride = (int64_t)gridDim.y * gridDim.x * NO * WAVE;
  f32x4* part = reinterpret_cast<f32x4*>(a.kpart) + grp * NO * WAVE + lane;
#pragma unroll
  for (int p = 0; p < NO / NOB; ++p) {
    if (p > 0) __syncthreads();   // the previous pass has read red
#pragma unroll
    for (int w = 0; w < NOB; ++w) {
      const int o = p * NOB + w;
      red[wave][w][lane] = acc[o / NMB][o % NMB];
    }
    __syncthreads();
    if (wave < NOB) {
      const int o = p * NOB + wave;
      f32x4 sum = red[0][wave][lane];
#pragma unroll
      for (int w = 1; w < kSkW; ++w) sum += red[w][wave][lane];
      if (ks > 1) part[blockIdx.z * zstride + (int64_t)o * WAVE] = sum;
      else skinny_finish<T, E, NMB>(a, M, N, tile0, m0, r, g, rsl, o, sum, p == 0 ? &pre : nullptr);
    }
  }
}

// Second kernel of a split launch (same grid x, y and block as gemm_skinny): adds the ks
// partial tiles of each output tile in split order and runs the row scale and epilogue.
template <typename T, Ep E, int NMB, int TPW>
__global__ __launch_bounds__(kSkW * WAVE) void skinny_reduce(int M, int N, int ks, EpArgs a) {
  constexpr int NO = TPW * NMB;
  constexpr int RPW = NMB * 16 / kSkW;
  __shared__ float rsl[NMB * 16];
  const int tile0 = blockIdx.x * TPW;
  const int m0 = blockIdx.y * (NMB * 16);
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r = lane & 15, g = lane >> 4;
  if (a.rs_ssp) {
    float4 ssr[RPW];
    skinny_scale_loads<NMB>(a, ssr, m0, M, wave, lane);
    skinny_scales<NMB>(a, ssr, rsl, wave, lane);
    __syncthreads();
  }
  const int64_t grp = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t zstride = (int64_t)gridDim.y * gridDim.x * NO * WAVE;
  const f32x4* part = reinterpret_cast<const f32x4*>(a.kpart) + grp * NO * WAVE + lane;
  for (int o = wave; o < NO; o += kSkW) {
    f32x4 sum = part[(int64_t)o * WAVE];
    for (int z = 1; z < ks; ++z) sum += part[z * zstride + (int64_t)o * WAVE];
    skinny_finish<T, E, NMB>(a, M, N, tile0, m0, r, g, rsl, o, sum, nullptr);
  }
}

// ------------------------------------------------------------------ tiled (prefill)
constexpr int TB = 128;   // tile rows (both operands)
constexpr int TK = 32;    // k per stage
constexpr int TPAD = 5;   // uint4 per LDS row (4 used + 1 pad)

template <typename T, Ep E>
__global__ __launch_bounds__(256) void gemm_tiled(const T* __restrict__ X, int64_t ldx, const T* __restrict__ W,
                                                  int M, int N, int K, EpArgs a) {
  __shared__ uint4 sW[2][TB][TPAD];
  __shared__ uint4 sX[2][TB][TPAD];
  const int n0 = blockIdx.x * TB;
  const int m0 = blockIdx.y * TB;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r = lane & 15, g = lane >> 4;
  const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;

  // global load assignment: 2 x 16B of each tile per thread. Activations: row lrow, k group lq.
  // Weights (tile-major): tile wt, row wr, k group 2 * (stage & 1) + wg, half wh, so that 32
  // consecutive threads read 512 contiguous bytes; they land in LDS row 16 wt + wr, slot 2 wg + wh.
  const T* wsrc[2];
  const T* xsrc[2];
  int lrow[2], lq[2], wrow[2], wq[2];
  const int ntiles = (N + 15) / 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * 256;
    lrow[i] = idx >> 2;
    lq[i] = idx & 3;
    xsrc[i] = X + (int64_t)min(m0 + lrow[i], M - 1) * ldx + lq[i] * 8;
    const int wr = idx & 15, wg = (idx >> 4) & 1, wh = (idx >> 5) & 1, wt = idx >> 6;
    wrow[i] = wt * 16 + wr;
    wq[i] = wg * 2 + wh;
    wsrc[i] = W + (int64_t)min(n0 / 16 + wt, ntiles - 1) * 16 * K + wh * 512 + (wg * 16 + wr) * 8;
  }
  uint4 rw[2], rx[2];
  auto gload = [&](int k0) {
    const int kw = k0 < K ? k0 : k0 - K;   // two-term X: columns K .. 2K-1 meet the same weights
    const int64_t wk = (int64_t)(kw >> 6) * 1024 + ((kw >> 5) & 1) * 256;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rw[i] = *reinterpret_cast<const uint4*>(wsrc[i] + wk);
      rx[i] = *reinterpret_cast<const uint4*>(xsrc[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sW[buf][wrow[i]][wq[i]] = rw[i];
      sX[buf][lrow[i]][lq[i]] = rx[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (a.x_split ? 2 * K : K) / TK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * TK);
    uint4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = sW[buf][wn + i * 16 + r][g];
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = sX[buf][wm + j * 16 + r][g];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bfr[j], acc[i][j]);
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn + i * 16 + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm + j * 16 + r;
      if (m < M) {
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        epilogue<T, E>(a, m, n, v);
      }
    }
  }
}

// ------------------------------------------------------------------ large (prefill)
// 256 x 256 output tile per workgroup of 8 waves (2 x 4), each wave 128 x 64 (8 x 4 MFMA
// tiles), both operands staged in LDS in the MFMA lane order: a 16-row group of a 64-wide k
// slice is one 2 KB block whose first (second) 1 KB holds k 16g..16g+7 (16g+8..16g+15) of
// row r for lane 16g + r; a stage is one of those 1 KB halves of every 16-row group of both
// operands (32 KB). Weights arrive in that order already (tile-major packing); activation
// rows are gathered in it. Every fragment read is one contiguous 1 KB ds_read_b128 per
// wavefront; per wave and stage: 16 fragment reads for 64 MFMAs.
constexpr int kBT = 256;                 // tile rows (both operands)
constexpr int kBK = 64;                  // k per stage

// Output tile of workgroup `pid`. Workgroups are dispatched to the 8 XCDs round-robin (pid
// mod 8), so XCD x gets a contiguous run of tile indices q (the runs' lengths differ by at
// most one when 8 does not divide the tile count); within the run, tiles are walked in groups
// of kGroupM row tiles, every column tile of the group before the next group. The ~32
// workgroups an XCD runs at once then cover about 4 row tiles x 8 column tiles and share their
// activation and weight slices in its L2, instead of 32 row tiles of one column tile (each
// activation slice read once per column tile). Groups of 4 measured ~5% faster than 8 on the
// encoder GEMMs at d 4096 and 2048 (16: ~6% slower).
constexpr int kGroupM = 4;
__device__ __forceinline__ void large_tile(int pid, int ntm, int ntn, int& tm, int& tn) {
  const int nt = ntm * ntn;
  const int x = pid % 8, i = pid / 8;
  const int per = nt / 8, rem = nt % 8;
  const int q = x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int span = kGroupM * ntn;                 // tiles of one group of row tiles
  const int first = (q / span) * kGroupM;
  const int gsize = min(ntm - first, kGroupM);
  const int r = q % span;
  tm = first + r % gsize;
  tn = r / gsize;
}

// Eight waves (2 x 4, each 128 rows x 64 features) rather than four (2 x 2, 128 x 128): two
// waves per SIMD hide each other's LDS waits and barriers (measured +7-13%, e.g. 1014 against
// 915 TFLOP/s at M 32768, N 2048, K 5632; the result is the same bit for bit).
// The operands move straight from global memory into LDS (global_load_lds: 16 bytes per
// lane, a wavefront fills 1 KB of LDS per instruction; no staging registers) over a ring of
// four stage buffers, so that a stage is requested three stages before it is multiplied
// (measured on MI355X: 770-920 TFLOP/s on the medium-LM prefill GEMMs against 550-610 for
// the same tiles staged through registers with one stage of lookahead). Weight instruction
// i of a stage copies tile i's half (contiguous in the tile-major layout); activation
// instruction i gathers 16-row block i: lane l reads 8 values of row l % 16 at k 16 (l / 16)
// + 8 h.
template <typename T, Ep E>
__global__ __launch_bounds__(512) void gemm_large(const T* __restrict__ X, int64_t ldx, const T* __restrict__ W,
                                                       int M, int N, int K, EpArgs a) {
  // four stage buffers as distinct objects, each [W 1024 uint4 | X 1024 uint4]: with the stage
  // loop unrolled by four every LDS read names its buffer, so the compiler knows which
  // outstanding copies it depends on
  __shared__ uint4 sb0[2048], sb1[2048], sb2[2048], sb3[2048];
  constexpr int NI = 4;    // feature tiles per wave (wave tile: 128 rows x 64 features)
  constexpr int CPW = 2;   // weight tiles (and row blocks) copied per wave and stage
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r = lane & 15, g = lane >> 4;
  const int wm = (wave >> 2) * 128;
  const int wn = (wave & 3) * 64;
  const int ntm = (M + kBT - 1) / kBT, ntn = (N + kBT - 1) / kBT;
  int tm, tn;
  large_tile(blockIdx.x, ntm, ntn, tm, tn);
  const int m0 = tm * kBT, n0 = tn * kBT;
  const int nkw = K / kBK;
  const int nk = 2 * (a.x_split ? 2 * nkw : nkw);   // half-slice stages (a multiple of 2)

  // wave w issues tiles / row blocks CPW w .. CPW w + CPW - 1 of each stage
  const T* wbase = W + (int64_t)(n0 / 16 + wave * CPW) * 16 * K + lane * 8;
  const int xrow0 = m0 + wave * CPW * 16 + r;
  const T* xbase = X + g * 16;
  // two-term X: the hi and lo stages of each k slice follow each other (hi 0, lo 0, hi 1, ...),
  // so the second copy of a weight slice comes from L2
  auto issue = [&](int st_, uint4* sb) {
    const int p = st_ >> 1, h = st_ & 1;
    const int kw = a.x_split ? p >> 1 : p;
    const int kt = a.x_split && (p & 1) ? nkw + kw : kw;   // X column slice (lo terms after the hi)
    uint4* d = sb + wave * CPW * 64;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const T* wsrc = wbase + (int64_t)i * 16 * K + h * 512 + (int64_t)kw * 1024;
      const int row = min(xrow0 + i * 16, M - 1);
      const T* xsrc = xbase + (int64_t)row * ldx + h * 8 + (int64_t)kt * kBK;
      __builtin_amdgcn_global_load_lds((const void*)wsrc, (__attribute__((address_space(3))) void*)(d + i * 64), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)xsrc, (__attribute__((address_space(3))) void*)(d + 1024 + i * 64),
                                       16, 0, 0);
    }
  };

  f32x4 acc[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage s: wait for this wave's copies of s (the two later stages, 2 CPW copies each, may
  // still be in flight), a bare barrier (the fence of __syncthreads would also wait for
  // them), then request stage s + 3 into the buffer stage s - 1 used, and multiply stage s
  auto stage = [&](int s, const uint4* cur, uint4* nxt) {
    // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at max
    if (s + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F78);        // vmcnt(8)
    else if (s + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 3 < nk) issue(s + 3, nxt);
    const uint4* sw = cur + (wn / 16) * 64;
    const uint4* sx = cur + 1024 + (wm / 16) * 64;
    uint4 af[NI], bfr[8];
#pragma unroll
    for (int i = 0; i < NI; ++i) af[i] = sw[i * 64 + lane];
#pragma unroll
    for (int j = 0; j < 8; ++j) bfr[j] = sx[j * 64 + lane];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bfr[j], acc[i][j]);
  };
  issue(0, sb0);
  if (1 < nk) issue(1, sb1);
  if (2 < nk) issue(2, sb2);
  for (int s = 0; s < nk; s += 4) {
    stage(s, sb0, sb3);
    if (s + 1 < nk) stage(s + 1, sb1, sb0);
    if (s + 2 < nk) stage(s + 2, sb2, sb1);
    if (s + 3 < nk) stage(s + 3, sb3, sb2);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = n0 + wn + i * 16 + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm + j * 16 + r;
      if (m < M) {
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        epilogue<T, E>(a, m, n, v);
      }
    }
  }
}

// Two-term X (each row K hi terms, then K lo terms): the tiles and copies of gemm_large, but a
// stage holds one weight half-slice and both terms' activation half-slices (48 KB), so every
// weight fragment read from LDS feeds the MFMAs of both terms: 64 MFMAs per wave, one barrier
// and 20 fragment reads per stage (two stages, two barriers and 24 reads before). Ring of
// three stages requested two ahead (144 KB of LDS).
template <typename T, Ep E>
__global__ __launch_bounds__(512) void gemm_large_x2(const T* __restrict__ X, int64_t ldx, const T* __restrict__ W,
                                                     int M, int N, int K, EpArgs a) {
  // [W 1024 uint4 | X hi 1024 uint4 | X lo 1024 uint4] each, distinct objects (see gemm_large)
  __shared__ uint4 sb0[3072], sb1[3072], sb2[3072];
  constexpr int NI = 4;
  constexpr int CPW = 2;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r = lane & 15, g = lane >> 4;
  const int wm = (wave >> 2) * 128;
  const int wn = (wave & 3) * 64;
  const int ntm = (M + kBT - 1) / kBT, ntn = (N + kBT - 1) / kBT;
  int tm, tn;
  large_tile(blockIdx.x, ntm, ntn, tm, tn);
  const int m0 = tm * kBT, n0 = tn * kBT;
  const int nkw = K / kBK;
  const int nk = 2 * nkw;   // half-slice stages

  const T* wbase = W + (int64_t)(n0 / 16 + wave * CPW) * 16 * K + lane * 8;
  const int xrow0 = m0 + wave * CPW * 16 + r;
  const T* xbase = X + g * 16;
  auto issue = [&](int st_, uint4* sb) {
    const int kw = st_ >> 1, h = st_ & 1;
    uint4* d = sb + wave * CPW * 64;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const T* wsrc = wbase + (int64_t)i * 16 * K + h * 512 + (int64_t)kw * 1024;
      const int row = min(xrow0 + i * 16, M - 1);
      const T* xsrc = xbase + (int64_t)row * ldx + h * 8 + (int64_t)kw * kBK;
      __builtin_amdgcn_global_load_lds((const void*)wsrc, (__attribute__((address_space(3))) void*)(d + i * 64), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)xsrc, (__attribute__((address_space(3))) void*)(d + 1024 + i * 64),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(xsrc + (int64_t)nkw * kBK),
                                       (__attribute__((address_space(3))) void*)(d + 2048 + i * 64), 16, 0, 0);
    }
  };

  f32x4 acc[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage s: wait for this wave's copies of s (the next stage's 3 CPW copies may still be in
  // flight), a bare barrier, request stage s + 2 into the buffer stage s - 1 used, multiply
  auto stage = [&](int s, const uint4* cur, uint4* nxt) {
    if (s + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
    else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 2 < nk) issue(s + 2, nxt);
    const uint4* sw = cur + (wn / 16) * 64;
    uint4 af[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) af[i] = sw[i * 64 + lane];
#pragma unroll
    for (int t = 0; t < 2; ++t) {   // hi, then lo terms of the rows
      const uint4* sx = cur + 1024 * (1 + t) + (wm / 16) * 64;
      uint4 bfr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bfr[j] = sx[j * 64 + lane];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bfr[j], acc[i][j]);
    }
  };
  issue(0, sb0);
  if (1 < nk) issue(1, sb1);
  for (int s = 0; s < nk; s += 3) {
    stage(s, sb0, sb2);
    if (s + 1 < nk) stage(s + 1, sb1, sb0);
    if (s + 2 < nk) stage(s + 2, sb2, sb1);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = n0 + wn + i * 16 + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm + j * 16 + r;
      if (m < M) {
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        epilogue<T, E>(a, m, n, v);
      }
    }
  }
}

// ------------------------------------------------------------------ mid (decode, M >= 256)
// Decode GEMMs with a few hundred rows and a wide output are MFMA work, not weight
// streaming: 128 x 128 output tile per workgroup of 4 waves (2 x 2, each 64 x 64 = 4 x 4 MFMA
// tiles), the LDS layout and copy scheme of gemm_large at half the tile (a stage is 16 KB:
// one k half of 8 weight tiles and 8 row blocks; a ring of four stages requested three ahead;
// 64 KB of LDS, two workgroups per CU), and the folded-norm row scale of the input rows.
// (A ring of eight stages measured no faster: a stage's time is not the copies' latency.)
constexpr int kMT = 128;

template <typename T, Ep E>
__global__ __launch_bounds__(256) void gemm_mid(const T* __restrict__ X, int64_t ldx, const T* __restrict__ W, int M,
                                                int N, int K, EpArgs a) {
  // [W 512 uint4 | X 512 uint4] each; distinct objects so that every LDS read names its stage
  __shared__ uint4 sb0[1024], sb1[1024], sb2[1024], sb3[1024];
  __shared__ float rsl[kMT];
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int r = lane & 15, g = lane >> 4;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int ntm = (M + kMT - 1) / kMT;
  const int tm = blockIdx.x % ntm, tn = blockIdx.x / ntm;
  const int m0 = tm * kMT, n0 = tn * kMT;
  const int nkw = K / 64;
  const int nk = 2 * (a.x_split ? 2 * nkw : nkw);   // half-slice stages

  // wave w copies weight tiles 2 w, 2 w + 1 and row blocks 2 w, 2 w + 1 of each stage
  const T* wbase = W + (int64_t)(n0 / 16 + wave * 2) * 16 * K + lane * 8;
  const int xrow0 = m0 + wave * 32 + r;
  const T* xbase = X + g * 16;
  auto issue = [&](int st_, uint4* sb) {
    const int kt = st_ >> 1, h = st_ & 1;
    const int kw = kt < nkw ? kt : kt - nkw;
    uint4* d = sb + wave * 2 * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const T* wsrc = wbase + (int64_t)i * 16 * K + h * 512 + (int64_t)kw * 1024;
      const int row = min(xrow0 + i * 16, M - 1);
      const T* xsrc = xbase + (int64_t)row * ldx + h * 8 + (int64_t)kt * 64;
      __builtin_amdgcn_global_load_lds((const void*)wsrc, (__attribute__((address_space(3))) void*)(d + i * 64), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)xsrc, (__attribute__((address_space(3))) void*)(d + 512 + i * 64),
                                       16, 0, 0);
    }
  };
  issue(0, sb0);
  if (1 < nk) issue(1, sb1);
  if (2 < nk) issue(2, sb2);

  // folded RMSNorm of the input rows (while the first stages are in flight): wave w owns rows
  // m0 + 32 w .. + 31
  if (a.rs_ssp) {
    for (int i = 0; i < 32; ++i) {
      const int m = min(m0 + wave * 32 + i, M - 1);
      float t = 0.f;
      for (int k = lane; k < a.rs_n; k += WAVE) t += a.rs_ssp[(int64_t)m * a.rs_n + k];
      t = wave_sum_dpp(t);
      if (lane == 0) rsl[wave * 32 + i] = rsqrtf(t / (float)a.rs_d + a.rs_eps);
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // stage s: this wave's copies of s have landed (the two later stages, 4 copies each, may be
  // in flight), a bare barrier (the fence of __syncthreads would also wait for them), request
  // stage s + 3 into the buffer stage s - 1 used, multiply stage s
  auto stage = [&](int s, const uint4* cur, uint4* nxt) {
    // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at max
    if (s + 2 < nk) __builtin_amdgcn_s_waitcnt(0x0F78);        // vmcnt(8)
    else if (s + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + 3 < nk) issue(s + 3, nxt);
    const uint4* sw = cur + (wn / 16) * 64;
    const uint4* sx = cur + 512 + (wm / 16) * 64;
    uint4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = sw[i * 64 + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = sx[j * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bfr[j], acc[i][j]);
  };
  for (int s = 0; s < nk; s += 4) {
    stage(s, sb0, sb3);
    if (s + 1 < nk) stage(s + 1, sb1, sb0);
    if (s + 2 < nk) stage(s + 2, sb2, sb1);
    if (s + 3 < nk) stage(s + 3, sb3, sb2);
  }
  __syncthreads();   // rsl
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wn + i * 16 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm + j * 16 + r;
      if (m < M && n < N) {
        const float sc = a.rs_ssp ? rsl[wm + j * 16 + r] : 1.f;
        float v[4] = {acc[i][j][0] * sc, acc[i][j][1] * sc, acc[i][j][2] * sc, acc[i][j][3] * sc};
        epilogue<T, E>(a, m, n, v);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32
template <Ep E>
__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ X, int64_t ldx,
                                                const float* __restrict__ W, int M, int N, int K, EpArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = N / 4;
  if (idx >= (int64_t)M * nq) return;
  const int m = (int)(idx / nq);
  const int n = (int)(idx % nq) * 4;
  const float* x = X + (int64_t)m * ldx;
  const float* w0 = W + (int64_t)n * K;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) {
    const float xv = x[k];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fmaf(xv, w0[(int64_t)i * K + k], v[i]);
  }
  epilogue<float, E>(a, m, n, v);
}

// RLT_GEMM_LARGE=0 sends prefill shapes to the 128 x 128 kernel instead (comparisons).
static bool large_gemm_enabled() {
  static const int state = [] {
    const char* env = getenv("RLT_GEMM_LARGE");
    return env && env[0] == '0' ? 0 : 1;
  }();
  return state == 1;
}

template <typename T, Ep E>
static void launch16(const EpArgs& a, const void* X, int64_t ldx, const void* W, int M, int N, int K,
                     hipStream_t st) {
  const T *x = (const T*)X, *w = (const T*)W;
  const int mid_tiles = ((M + kMT - 1) / kMT) * ((N + kMT - 1) / kMT);
  if (M >= 2 * kMT && M <= kSkinnyMaxRows && mid_tiles >= 128 && K % 64 == 0 && !a.row_invariant && !a.fold_zb) {
    // a few hundred rows and a wide output: MFMA-bound tiles (measured on MI355X on the
    // medium-LM shapes: M 512, N 6144, K 2048 in 34 us against 54 us for the streaming
    // kernel below; with fewer than 128 tiles the streaming kernel stays faster)
    const int nt = mid_tiles;
    hipLaunchKernelGGL((gemm_mid<T, E>), dim3(nt), dim3(256), 0, st, x, ldx, w, M, N, K, a);
  } else if (M <= kSkinnyMaxRows || a.fold_zb || a.rs_ssp || a.row_invariant) {
    // Tiles per workgroup (TPW), row blocks (NMB) and K splits (S) from a cost model fitted to
    // MI355X measurements of this kernel: one workgroup per CU at a time, each round of up to
    // 256 workgroups costs a memory latency (~70 KB of per-CU transfer time) plus its
    // workgroup's bytes (TPW weight tiles + the X rows it reads, over its K range) at the
    // per-CU rate.
    const dim3 blk(kSkW * WAVE);
    const int64_t xs = a.x_split ? 2 : 1, e = sizeof(T);
    const int nch = K / 64;
    // (4 x 4 tiles measured slower than 4 x 2 with two row blocks at 64 two-term rows: four
    // reduction passes and 160 registers)
    static const int cand[][2] = {{1, 1}, {1, 2}, {1, 4}, {2, 1}, {2, 2}, {2, 4}, {4, 1}, {4, 2}};
    int best_t = 1, best_n = 1, best_s = 1;
    int64_t best_cost = -1;
    auto fits = [&](int tpw, int nmb, int ks) {
      if (tpw > 1 && N % (16 * tpw) != 0) return false;   // one tile per workgroup covers a ragged N
      if (ks == 1) return true;
      // split launches: row-invariant arithmetic keeps one K order; every split gets a chunk per wave
      if (a.row_invariant || !a.kpart || nch % ks != 0 || nch / ks < kSkW) return false;
      const int64_t gx = (N + 16 * tpw - 1) / (16 * tpw), gy = (M + 16 * nmb - 1) / (16 * nmb);
      return (int64_t)ks * gy * gx * tpw * nmb * 256 <= a.kpart_n;
    };
    for (const auto& c : cand) {
      const int tpw = c[0], nmb = c[1];
      for (int ks = 1; ks <= kMaxKSplit; ks *= 2) {
        if (!fits(tpw, nmb, ks)) continue;
        const int64_t wgs = (int64_t)((N + 16 * tpw - 1) / (16 * tpw)) * ((M + 16 * nmb - 1) / (16 * nmb)) * ks;
        const int64_t rows = std::min(16 * nmb, M);
        const int64_t bytes = ((int64_t)tpw * 16 * K * e + rows * K * e * xs) / ks;
        int64_t cost = ((wgs + 255) / 256) * (70 * 1024 + bytes);
        // a split launch adds the reduce kernel: a dependent launch and its memory latency, and
        // the partial tiles written and read back
        if (ks > 1) cost += 2 * 70 * 1024 + (int64_t)(ks + 1) * tpw * nmb * 1024;
        if (best_cost < 0 || cost < best_cost) {
          best_cost = cost;
          best_t = tpw;
          best_n = nmb;
          best_s = ks;
        }
      }
    }
    const int ov_t = a.tile_ov[0], ov_n = a.tile_ov[1], ov_s = a.tile_ov[2];
    bool ov_ok = false;   // only the compiled tile shapes
    for (const auto& c : cand) ov_ok = ov_ok || (c[0] == ov_t && c[1] == ov_n);
    if (ov_ok && ov_s >= 1 && ov_s <= kMaxKSplit && fits(ov_t, ov_n, ov_s)) {
      best_t = ov_t;
      best_n = ov_n;
      best_s = ov_s;
    }
    const dim3 grid((N + 16 * best_t - 1) / (16 * best_t), (M + 16 * best_n - 1) / (16 * best_n), best_s);
    // nontemporal weight loads only when no other row block of this launch reads the same
    // tiles (measured at the paper shape: B 1 5.52 -> 5.20 ms per step; at B 64, with two row
    // blocks, the hint made the second read miss the cache: 4% slower)
    const bool nt = a.stream_w && grid.y == 1 && a.x_split;
#define RLT_SKINNY(NMB_, TPW_)                                                                                   \
  if (best_n == NMB_ && best_t == TPW_) {                                                                        \
    if (best_s > 1) {                                                                                            \
      if (nt) hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, true, true, true>), grid, blk, 0, st, x, ldx, w, M, N, K, a); \
      else if (a.x_split) hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, true, false, true>), grid, blk, 0, st, x, ldx, w, M, N, K, a); \
      else hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, false, false, true>), grid, blk, 0, st, x, ldx, w, M, N, K, a); \
      hipLaunchKernelGGL((skinny_reduce<T, E, NMB_, TPW_>), dim3(grid.x, grid.y), blk, 0, st, M, N, best_s, a);  \
    } else if (nt) hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, true, true>), grid, blk, 0, st, x, ldx, w, M, N, K, a); \
    else if (a.x_split) hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, true>), grid, blk, 0, st, x, ldx, w, M, N, K, a); \
    else hipLaunchKernelGGL((gemm_skinny<T, E, NMB_, TPW_, false>), grid, blk, 0, st, x, ldx, w, M, N, K, a);   \
    return;                                                                                                      \
  }
    RLT_SKINNY(1, 1) RLT_SKINNY(2, 1) RLT_SKINNY(4, 1) RLT_SKINNY(1, 2) RLT_SKINNY(2, 2) RLT_SKINNY(4, 2)
    RLT_SKINNY(1, 4) RLT_SKINNY(2, 4)
#undef RLT_SKINNY
  } else if (large_gemm_enabled() && K % kBK == 0) {
    const int nt = ((M + kBT - 1) / kBT) * ((N + kBT - 1) / kBT);
    if (a.x_split) hipLaunchKernelGGL((gemm_large_x2<T, E>), dim3(nt), dim3(512), 0, st, x, ldx, w, M, N, K, a);
    else hipLaunchKernelGGL((gemm_large<T, E>), dim3(nt), dim3(512), 0, st, x, ldx, w, M, N, K, a);
  } else {
    hipLaunchKernelGGL((gemm_tiled<T, E>), dim3((N + TB - 1) / TB, (M + TB - 1) / TB), dim3(256), 0, st, x, ldx, w,
                       M, N, K, a);
  }
}

template <Ep E>
static void launch(Dt dt, const EpArgs& a, const void* X, int64_t ldx, const void* W, int M, int N, int K,
                   hipStream_t st) {
  if (M <= 0 || N <= 0) return;
  if (dt == Dt::F32) {
    const int64_t total = (int64_t)M * (N / 4);
    const int blocks = (int)((total + 255) / 256);
    hipLaunchKernelGGL(gemm_f32<E>, dim3(blocks), dim3(256), 0, st, (const float*)X, ldx, (const float*)W, M, N, K,
                       a);
  } else if (dt == Dt::BF16) {
    launch16<bf16_t, E>(a, X, ldx, W, M, N, K, st);
  } else {
    launch16<f16_t, E>(a, X, ldx, W, M, N, K, st);
  }
}

void gemm(Dt dt, Ep ep, const EpArgs& a, const void* X, int64_t ldx, const void* W, int M, int N, int K,
          hipStream_t st) {
  switch (ep) {
    case Ep::StoreAct: launch<Ep::StoreAct>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::StoreF32: launch<Ep::StoreF32>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::Residual: launch<Ep::Residual>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::SwiGLU: launch<Ep::SwiGLU>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::QKV: launch<Ep::QKV>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::RopeQ: launch<Ep::RopeQ>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::MemKV: launch<Ep::MemKV>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::Merge: launch<Ep::Merge>(dt, a, X, ldx, W, M, N, K, st); break;
    case Ep::Bias: launch<Ep::Bias>(dt, a, X, ldx, W, M, N, K, st); break;
  }
}

}  // namespace rlt
