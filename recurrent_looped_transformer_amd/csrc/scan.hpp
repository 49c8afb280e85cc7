// Persistent decoder-scan kernel: parameters and launcher.
//
// One cooperative launch runs every decoder transition of a scan (positions
// start+1 .. start+T of all B sequences): per pass the merge, then per decoder
// layer the SWA, cross-attention and FFN sublayers, each a grid-wide phase
// separated by a hierarchical barrier. Activations that cross workgroups are
// written and read with device-scope (SC1) cache policy, so no phase needs an
// L2 writeback or invalidate.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace rlt {

struct ScanLayer {
  const bf16_t *wqkv, *wo, *xq, *xo, *w13, *w2;   // packed bf16 weights
  const float *g1, *g2, *g3;                       // pre-norm gains of the SWA, cross and FFN sublayers
  const float* gnext;                              // gain of the norm that consumes this layer's output
  const bf16_t *mk, *mv;                           // memory of this layer's group, [B][H][Tm][dh]
  bf16_t *rk, *rv;                                 // this layer's ring, [B][H][R][dh]
};

struct ScanParams {
  int B, d, hd, H, dh, f, L, W, R, Tm, variant, chunk, P;
  int ngroups;                // 1: one group of all blocks; 8*k: k blocks per CU, groups confined to one XCD
  int cpx;                    // CUs per XCD
  float alpha, eps, scale;
  const bf16_t* wsr;          // [2d][d] rows (2j, 2j+1) = (W_g,r row j, W_s row j)
  const float* ns;            // RMSNorm_s gain
  const float* g_first;       // gain of the first layer's first norm (RLT-0 entry, or merge output)
  const float* e;             // [B][Tm][d] encoder outputs
  const float* gpre;          // [B][Tm][d] W_g,e e_t + b_g
  float* s;                   // [B][d] s_t of the last consumed position
  float* rho;                 // [B][d] feedback register (s_{t-1} for RLT-1)
  bf16_t* rhob;               // [B][d] bf16(rho * ns)
  float* rhoss;               // [d/16][B] sum-of-squares partials of rho
  const float2* rope;         // [Tm+1][dh/2]
  float* z[2];                // [B*P][d] residual stream, ping-pong by pass parity
  bf16_t* zb[2];              // [B*P][d] bf16(z * gain of the consuming norm)
  float* ssp[2];              // [d/8][B*P] sum-of-squares partials of z
  bf16_t *q, *ao, *hid;       // [B*P][hd], [B*P][hd], [B*P][f]
  float* sall;                // [B][Tm][d] s_t of every position (readout input)
  int start, T;
  unsigned* bar;              // barrier words, zeroed before the launch
  const ScanLayer* layer;     // [L] in device memory
};

constexpr int kScanThreads = 256;
constexpr int kBarWords = 64 * 52;   // per-XCD counters, top counter, release flag, abort, group member flags

// Returns hipSuccess or the launch error; *grid_out receives the grid size used.
hipError_t launch_scan(const ScanParams& p, int* grid_out, hipStream_t st);
int scan_cus();
bool scan_supported(int dh, int rows, int d, int hd, int f, int Tm, int L);
int scan_lds_bytes(int Tm, int W, int R, int dh);

}  // namespace rlt
