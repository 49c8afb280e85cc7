// Attention of one query row per (sequence, head, query index) over a contiguous
// range of positions of a key/value store: the decoder's sliding-window
// self-attention over its ring (keys max(1, t-W+1)..t, greeksharifa summary
// §2.1, jiphyeonjeon review §3.3), the cross-attention to the prefix memory
// M_<=t (keys 1..t, greeksharifa summary §2.2, §2.4) and the encoder's
// attention over its cache.
//
// One workgroup (256 threads) per (head, query row). A group of DH/VEC lanes
// owns one key (16-byte loads), so a wave reads whole contiguous key rows.
// Pass 1 writes the scaled scores to LDS, pass 2 takes max / exp / sum, pass 3
// accumulates p_j v_j per lane group and reduces the groups through LDS. Keys
// and values are each read once from HBM.
#include "common.hpp"
#include "ops.hpp"

namespace rlt {

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_decode_k(AttnArgs a) {
  extern __shared__ float smem[];          // [n] scores, then [256/G][DH] partials
  __shared__ float red[16];
  constexpr int VEC = Elem<T>::VEC;
  constexpr int G = DH / VEC;              // lanes per key
  constexpr int NG = 256 / G;              // keys in flight per block
  const int h = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / a.nq, qi = row % a.nq;
  const int pos = a.pos0 + 1 + qi;
  const int lo = a.window > 0 ? max(1, pos - a.window + 1) : 1;
  const int n = pos - lo + 1;
  const int tid = threadIdx.x, gi = tid / G, gl = tid % G;

  const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)row * a.ldq + h * DH + gl * VEC;
  float qv[VEC];
  load16(qp, qv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] *= a.scale;
  const int64_t hb = (int64_t)b * a.kv_bstride + (int64_t)h * a.cap * DH + gl * VEC;
  const T* kb = reinterpret_cast<const T*>(a.k) + hb;
  const T* vb = reinterpret_cast<const T*>(a.v) + hb;

  float* sc = smem;
  for (int j = gi; j < n; j += NG) {
    const int p = lo + j;
    const int slot = a.ring ? (p - 1) % a.cap : p - 1;
    float kv[VEC];
    load16(kb + (int64_t)slot * DH, kv);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = fmaf(qv[e], kv[e], dot);
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, WAVE);
    if (gl == 0) sc[j] = dot;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < n; j += 256) mx = fmaxf(mx, sc[j]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = tid; j < n; j += 256) {
    const float e = __expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  sum = block_sum(sum, red);   // ends with a barrier: sc[] final for everyone
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int j = gi; j < n; j += NG) {
    const int p = lo + j;
    const int slot = a.ring ? (p - 1) % a.cap : p - 1;
    float vv[VEC];
    load16(vb + (int64_t)slot * DH, vv);
    const float w = sc[j];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w, vv[e], acc[e]);
  }
  __syncthreads();   // scores no longer needed: reuse LDS for partials
  float* part = smem;   // [NG][DH]
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[gi * DH + gl * VEC + e] = acc[e];
  __syncthreads();
  if (tid < DH) {
    float s = 0.f;
    for (int gg = 0; gg < NG; ++gg) s += part[gg * DH + tid];
    T* op = reinterpret_cast<T*>(a.out) + (int64_t)row * a.ldo + h * DH + tid;
    Elem<T>::st(op, s / sum);
  }
}

template <typename T, int DH>
static void launch_attn(const AttnArgs& a, hipStream_t st) {
  const int maxn = a.window > 0 ? a.window : a.pos0 + a.nq;
  constexpr int VEC = Elem<T>::VEC;
  constexpr int NG = 256 / (DH / VEC);
  const size_t lds = sizeof(float) * (size_t)max(maxn, NG * DH);
  hipLaunchKernelGGL((attn_decode_k<T, DH>), dim3(a.H, a.B * a.nq), dim3(256), lds, st, a);
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
  else attn_dispatch<bf16_t>(a, st);
}

}  // namespace rlt
