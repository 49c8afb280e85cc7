// Row-wise and elementwise kernels: RMSNorm (wavefront per row), embedding
// gather, rotary table, row copies, state broadcast, readout log-probability,
// and weight packing into the library layout.
#include <algorithm>

#include "common.hpp"
#include "ops.hpp"

namespace rlt {

// out[m, :] = act(x[m, :] / sqrt(mean(x^2) + eps) * gain); one wavefront per row. Rows up to
// 64 * 4 * kRmsVec features are read once into registers with every load in flight together;
// longer rows take a second, streaming pass.
constexpr int kRmsVec = 16;
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_k(const float* __restrict__ x, RowMap xm,
                                                 const float* __restrict__ gain, T* __restrict__ out,
                                                 int64_t ldo, int rows, int d, float eps, int64_t lo_off) {
  const int row = blockIdx.x * 4 + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (row >= rows) return;
  const float* xr = x + xm.off(row);
  float4 v[kRmsVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = (lane + WAVE * i) * 4;
    v[i] = c < d ? *reinterpret_cast<const float4*>(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  for (int c = (lane + WAVE * kRmsVec) * 4; c < d; c += WAVE * 4) {
    const float4 u = *reinterpret_cast<const float4*>(xr + c);
    ss += u.x * u.x + u.y * u.y + u.z * u.z + u.w * u.w;
  }
  ss = wave_sum_dpp(ss);
  const float inv = gain ? rsqrtf(ss / (float)d + eps) : 1.f;
  T* o = out + (int64_t)row * ldo;
  auto put = [&](int c, float4 u) {
    const float4 gv = gain ? *reinterpret_cast<const float4*>(gain + c) : make_float4(1.f, 1.f, 1.f, 1.f);
    store_act<T>(o + c, lo_off, u.x * inv * gv.x);
    store_act<T>(o + c + 1, lo_off, u.y * inv * gv.y);
    store_act<T>(o + c + 2, lo_off, u.z * inv * gv.z);
    store_act<T>(o + c + 3, lo_off, u.w * inv * gv.w);
  };
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = (lane + WAVE * i) * 4;
    if (c < d) put(c, v[i]);
  }
  for (int c = (lane + WAVE * kRmsVec) * 4; c < d; c += WAVE * 4) put(c, *reinterpret_cast<const float4*>(xr + c));
}

void rmsnorm(Dt dt, const float* x, RowMap xm, const float* gain, void* out, int64_t ldo, int rows, int d,
             float eps, hipStream_t st, int64_t out_split) {
  if (rows <= 0) return;
  const dim3 grid((rows + 3) / 4);
  if (dt == Dt::F32)
    hipLaunchKernelGGL(rmsnorm_k<float>, grid, dim3(256), 0, st, x, xm, gain, (float*)out, ldo, rows, d, eps,
                       (int64_t)0);
  else if (dt == Dt::BF16)
    hipLaunchKernelGGL(rmsnorm_k<bf16_t>, grid, dim3(256), 0, st, x, xm, gain, (bf16_t*)out, ldo, rows, d, eps,
                       out_split);
  else
    hipLaunchKernelGGL(rmsnorm_k<f16_t>, grid, dim3(256), 0, st, x, xm, gain, (f16_t*)out, ldo, rows, d, eps,
                       out_split);
}

template <typename T>
__global__ void embed_k(const int32_t* __restrict__ tok, const T* __restrict__ emb, float* __restrict__ h,
                        RowMap hm, int rows, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = d / 4;
  if (idx >= (int64_t)rows * per) return;
  const int m = (int)(idx / per), c = (int)(idx % per) * 4;
  const T* e = emb + (int64_t)tok[m] * d + c;
  float* o = h + hm.off(m) + c;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = Elem<T>::ld(e + i);
}

void embed(Dt dt, const int32_t* tok, const void* emb, float* h, RowMap hm, int rows, int d, hipStream_t st) {
  if (rows <= 0) return;
  const int64_t total = (int64_t)rows * (d / 4);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dt == Dt::F32) hipLaunchKernelGGL(embed_k<float>, grid, dim3(256), 0, st, tok, (const float*)emb, h, hm, rows, d);
  else if (dt == Dt::BF16)
    hipLaunchKernelGGL(embed_k<bf16_t>, grid, dim3(256), 0, st, tok, (const bf16_t*)emb, h, hm, rows, d);
  else hipLaunchKernelGGL(embed_k<f16_t>, grid, dim3(256), 0, st, tok, (const f16_t*)emb, h, hm, rows, d);
}

// angle p * base^(-2i/dh), evaluated in double precision, stored as float (cos, sin)
__global__ void rope_table_k(float2* tab, int npos, int dh, double base) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = dh / 2;
  if (idx >= (int64_t)npos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double theta = pow(base, -2.0 * (double)i / (double)dh);
  const double ang = (double)p * theta;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

void rope_table(float2* tab, int npos, int dh, float base, hipStream_t st) {
  const int64_t total = (int64_t)npos * (dh / 2);
  hipLaunchKernelGGL(rope_table_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, tab, npos, dh,
                     (double)base);
}

__global__ void copy_rows_k(const float* __restrict__ src, RowMap sm, float* __restrict__ dst, RowMap dm, int rows,
                            int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = d / 4;
  if (idx >= (int64_t)rows * per) return;
  const int m = (int)(idx / per), c = (int)(idx % per) * 4;
  *reinterpret_cast<float4*>(dst + dm.off(m) + c) = *reinterpret_cast<const float4*>(src + sm.off(m) + c);
}

void copy_rows(const float* src, RowMap sm, float* dst, RowMap dm, int rows, int d, hipStream_t st) {
  if (rows <= 0) return;
  const int64_t total = (int64_t)rows * (d / 4);
  hipLaunchKernelGGL(copy_rows_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, sm, dst, dm, rows, d);
}

__global__ void copy_rows_at_k(const float* __restrict__ src, RowMap sm, float* __restrict__ dst, RowMap dm,
                               const int* __restrict__ col_dev, int64_t col_stride, int rows, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = d / 4;
  if (idx >= (int64_t)rows * per) return;
  const int m = (int)(idx / per), c = (int)(idx % per) * 4;
  const int64_t o = dm.off(m) + (int64_t)col_dev[0] * col_stride + c;
  *reinterpret_cast<float4*>(dst + o) = *reinterpret_cast<const float4*>(src + sm.off(m) + c);
}

void copy_rows_at(const float* src, RowMap sm, float* dst, RowMap dm, const int* col_dev, int64_t col_stride,
                  int rows, int d, hipStream_t st) {
  if (rows <= 0) return;
  const int64_t total = (int64_t)rows * (d / 4);
  hipLaunchKernelGGL(copy_rows_at_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, sm, dst, dm,
                     col_dev, col_stride, rows, d);
}

__global__ void set_scan_pos_k(int* p, int pos, int col) {
  p[0] = pos;
  p[1] = col;
}
__global__ void advance_scan_pos_k(int* p, int np) {
  p[0] += np;
  p[1] += np;
}
void set_scan_pos(int* p, int pos, int col, hipStream_t st) {
  hipLaunchKernelGGL(set_scan_pos_k, dim3(1), dim3(1), 0, st, p, pos, col);
}
void advance_scan_pos(int* p, int np, hipStream_t st) {
  hipLaunchKernelGGL(advance_scan_pos_k, dim3(1), dim3(1), 0, st, p, np);
}

// Grid-stride (a dispatch holds fewer than 2^32 work-items, and ring buffers of large
// states exceed that many words): 16-byte stores over the aligned body, words at the ends.
__global__ void fill_zero_k(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t mis = (int64_t)((16 - ((uintptr_t)p & 15)) & 15) / 4;   // words before a 16-byte boundary
  const int64_t head = mis < n ? mis : n;
  const int64_t n4 = (n - head) / 4;
  uint4* q = reinterpret_cast<uint4*>(p + head);
  for (int64_t i = t; i < n4; i += stride) q[i] = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = t; i < head; i += stride) p[i] = 0u;
  for (int64_t i = head + 4 * n4 + t; i < n; i += stride) p[i] = 0u;
}

void fill_zero_u32(void* p, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = std::min<int64_t>((n / 4 + 255) / 256 + 1, 16384);
  hipLaunchKernelGGL(fill_zero_k, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, n);
}

__global__ void broadcast_row_k(const float* __restrict__ s0, float* __restrict__ s, int B, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * d) return;
  s[idx] = s0[idx % d];
}

void broadcast_row(const float* s0, float* s, int B, int d, hipStream_t st) {
  const int64_t total = (int64_t)B * d;
  hipLaunchKernelGGL(broadcast_row_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, s0, s, B, d);
}

// Rows at different positions: dst[b] <- src[b] (or the one vector src when src_ld == 0) for
// the rows with mask[b] != 0; other rows untouched.
__global__ void masked_rows_k(const float* __restrict__ src, int64_t src_ld, float* __restrict__ dst,
                              const int* __restrict__ mask, int B, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * d) return;
  const int b = (int)(idx / d), c = (int)(idx % d);
  if (mask[b]) dst[idx] = src[(int64_t)b * src_ld + c];
}

void masked_rows(const float* src, int64_t src_ld, float* dst, const int* mask, int B, int d, hipStream_t st) {
  const int64_t total = (int64_t)B * d;
  hipLaunchKernelGGL(masked_rows_k, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, src_ld, dst,
                     mask, B, d);
}

// out[b] = keep[b] ? 0 : tok[b]: the token of a row that does not move is never read as an id
__global__ void active_tokens_k(const int32_t* __restrict__ tok, const int* __restrict__ keep,
                                int32_t* __restrict__ out, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) out[b] = keep[b] ? 0 : tok[b];
}

void active_tokens(const int32_t* tok, const int* keep, int32_t* out, int B, hipStream_t st) {
  hipLaunchKernelGGL(active_tokens_k, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, tok, keep, out, B);
}

// dst row (row_off + row_stride * perm(j)) <- src row j, columns [col0, col0 + cols) -> [dst_col0, ...)
// RopeRows: within each head of dh rows, rotate-half pair (i, i + dh/2) lands on rows (2i, 2i + 1).
template <typename T>
__global__ void pack_k(const float* __restrict__ src, int64_t src_ld, int64_t col0, T* __restrict__ dst,
                       int64_t dst_ld, int64_t dst_col0, int rows, int cols, int kind, int dh, int row_stride,
                       int row_off, int tiles) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * cols) return;
  const int j = (int)(idx / cols), c = (int)(idx % cols);
  int pj = j;
  if (kind == (int)Pack::RopeRows) {
    const int h = j / dh, w = j % dh, half = dh / 2;
    pj = h * dh + (w < half ? 2 * w : 2 * (w - half) + 1);
  }
  const int64_t drow = (int64_t)row_off + (int64_t)row_stride * pj;
  const int64_t o = tiles ? tile_major_off(drow, dst_col0 + c, dst_ld) : drow * dst_ld + dst_col0 + c;
  Elem<T>::st(dst + o, src[(int64_t)j * src_ld + col0 + c]);
}

void pack_matrix(Dt dt, const float* src, int64_t src_ld, int64_t col0, void* dst, int64_t dst_ld, int64_t dst_col0,
                 int rows, int cols, Pack kind, int dh, int row_stride, int row_off, bool tiles, hipStream_t st) {
  const int64_t total = (int64_t)rows * cols;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dt == Dt::F32)
    hipLaunchKernelGGL(pack_k<float>, grid, dim3(256), 0, st, src, src_ld, col0, (float*)dst, dst_ld, dst_col0, rows,
                       cols, (int)kind, dh, row_stride, row_off, 0);
  else if (dt == Dt::BF16)
    hipLaunchKernelGGL(pack_k<bf16_t>, grid, dim3(256), 0, st, src, src_ld, col0, (bf16_t*)dst, dst_ld, dst_col0,
                       rows, cols, (int)kind, dh, row_stride, row_off, tiles ? 1 : 0);
  else
    hipLaunchKernelGGL(pack_k<f16_t>, grid, dim3(256), 0, st, src, src_ld, col0, (f16_t*)dst, dst_ld, dst_col0,
                       rows, cols, (int)kind, dh, row_stride, row_off, tiles ? 1 : 0);
}


// ------------------------------------------------------------------ digest
// Order-independent 64-bit digest of a buffer of 64-bit words: the sum (mod 2^64) of
// splitmix64-finalised (word ^ index * golden-ratio constant) values (the finaliser of
// Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__global__ __launch_bounds__(256) void digest_k(const uint64_t* __restrict__ w, int64_t n, unsigned long long* out) {
  uint64_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    acc += mix64(w[i] ^ ((uint64_t)i * 0x9E3779B97F4A7C15ull));
  __shared__ uint64_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicAdd(out, (unsigned long long)red[0]);
}

void digest64(const void* p, int64_t n_words, uint64_t* out_dev, hipStream_t st) {
  fill_zero_u32(out_dev, 2, st);
  if (n_words <= 0) return;
  const int64_t blocks = std::min<int64_t>((n_words + 255) / 256, 4096);
  hipLaunchKernelGGL(digest_k, dim3((unsigned)blocks), dim3(256), 0, st, (const uint64_t*)p, n_words,
                     (unsigned long long*)out_dev);
}

}  // namespace rlt
