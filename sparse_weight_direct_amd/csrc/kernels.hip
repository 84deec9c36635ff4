// gfx950 kernels: sparse direct convolution and its dense direct baseline.
//
// One workgroup = 8 wavefronts = one tile of 64*K consecutive extended output positions
// (see plan.h) x one group of output channels.  Steps per workgroup:
//   1. a small row table maps each staged phase row to its image row (or -1 = zero row);
//   2. for each chunk of Cc input channels: all 512 threads copy the phase rows of the
//      chunk from HBM into LDS, zero-filling padding (coalesced along x), barrier;
//   3. each wavefront walks the non-zeros of its output-channel slots for that chunk.
//      A non-zero is wave-uniform (scalar loads of {enc, value}); per non-zero each lane
//      does one address add, K LDS reads 64 words apart and K fp32 FMAs into registers;
//   4. after the last chunk, coalesced NCHW stores of the valid positions; slots of
//      channels without non-zeros store exact zeros.
// The tiling with a halo staged once per block and reused by every output channel, the
// packed per-non-zero word and the per-thread register accumulators follow Tuteja et al.,
// Sec. 5.1-5.5; the wave-uniform weight broadcast with lanes over consecutive output
// positions follows the thread-per-output dataflow of "Escoin" (dataflow section).
#include <hip/hip_runtime.h>

#include "plan.h"

namespace sc {

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that consecutive
// logical ids (the channel groups of one tile, then neighbouring tiles that share halo
// rows) run on the same XCD and hit its L2.
__device__ __forceinline__ int xcd_logical(int b, int nb) {
  const int q = nb >> 3, rmd = nb & 7;
  const int xcd = b & 7, k = b >> 3;
  return xcd < rmd ? xcd * (q + 1) + k : rmd * (q + 1) + (xcd - rmd) * q + k;
}

// Row table: for staged phase row j of phase py, the word offset n*C*H*W + y*W of the
// input row it holds, or -1 when the row is padding or past the last image.
__device__ __forceinline__ void build_row_table(const KArgs& a, int t0, int* rowinfo) {
  for (int i = threadIdx.x; i < a.st * a.NRmax; i += kThreads) {
    const int py = i / a.NRmax;
    const int j = i - py * a.NRmax;
    const int T = t0 + j;
    const int n = T / a.HYp;
    const int y = (T - n * a.HYp) * a.st + py - a.pad;
    rowinfo[i] = (n < a.N && y >= 0 && y < a.H) ? (n * a.C * a.H + y) * a.W : -1;
  }
}

// Copy channels [c0, c0+cc) of the tile's phase rows into LDS (zero outside the image).
__device__ __forceinline__ void stage_chunk(const KArgs& a, const float* __restrict__ x,
                                            const int* rowinfo, float* lds, int c0, int cc) {
  const int SC = a.st * a.Pp;  // padded columns covered by one phase row set
  const int HW = a.H * a.W;
  if (SC <= kThreads) {
    const int rows_pp = kThreads / SC;
    const int rsub = threadIdx.x / SC;
    const int col = threadIdx.x - rsub * SC;
    if (rsub >= rows_pp) return;
    const int px = col % a.st, xq = col / a.st;
    const int xg = col - a.pad;
    const bool xok = xg >= 0 && xg < a.W;
    const int ldscol = px * a.PH + xq;
    for (int cl = 0; cl < cc; cl++) {
      const float* xc = x + (long long)(c0 + cl) * HW + (xok ? xg : 0);
      float* lc = lds + cl * a.CHS + ldscol;
      for (int py = 0; py < a.st; py++) {
        const int* ri = rowinfo + py * a.NRmax;
        float* lp = lc + py * a.st * a.PH;
#pragma unroll 4
        for (int j = rsub; j < a.NRmax; j += rows_pp) {
          const int r = ri[j];
          lp[j * a.Pp] = (xok && r >= 0) ? xc[r] : 0.0f;
        }
      }
    }
  } else {
    for (int col = threadIdx.x; col < SC; col += kThreads) {
      const int px = col % a.st, xq = col / a.st;
      const int xg = col - a.pad;
      const bool xok = xg >= 0 && xg < a.W;
      const int ldscol = px * a.PH + xq;
      for (int cl = 0; cl < cc; cl++) {
        const float* xc = x + (long long)(c0 + cl) * HW + (xok ? xg : 0);
        float* lc = lds + cl * a.CHS + ldscol;
        for (int py = 0; py < a.st; py++) {
          const int* ri = rowinfo + py * a.NRmax;
          float* lp = lc + py * a.st * a.PH;
          for (int j = 0; j < a.NRmax; j++) {
            const int r = ri[j];
            lp[j * a.Pp] = (xok && r >= 0) ? xc[r] : 0.0f;
          }
        }
      }
    }
  }
}

// Output word offset (without the channel term) of each of the lane's K positions, or -1.
template <int K>
__device__ __forceinline__ void output_bases(const KArgs& a, int I0, int lane, int (&ob)[K]) {
#pragma unroll
  for (int b = 0; b < K; b++) {
    const long long I = (long long)I0 + lane + 64 * b;
    ob[b] = -1;
    if (I < a.ext_total) {
      const int Ii = (int)I;
      const int n = Ii / a.img_ext;
      const int rem = Ii - n * a.img_ext;
      const int e = rem / a.Pp;
      const int f = rem - e * a.Pp;
      if (e < a.E && f < a.F) ob[b] = (n * a.M * a.E + e) * a.F + f;
    }
  }
}

// One non-zero: K FMAs of the wave-uniform weight into the lane's K positions.
template <int K>
__device__ __forceinline__ void fma_entry(float (&acc)[K], const float* lane_lds, uint2 e) {
  const float w = __uint_as_float(e.y);
  const float* p = lane_lds + e.x;
#pragma unroll
  for (int b = 0; b < K; b++) acc[b] = fmaf(w, p[64 * b], acc[b]);
}

// Pointers are separate restrict-qualified arguments: the compiler may then read the
// read-only streams with scalar loads (one s_load_dwordx16 brings 8 non-zeros).
template <int K, int OCW>
__global__ __launch_bounds__(kThreads) void sparse_direct_fwd(
    const KArgs a, const float* __restrict__ x, float* __restrict__ y,
    const uint2* __restrict__ ent, const int2* __restrict__ seg,
    const int* __restrict__ slot_row) {
  extern __shared__ float lds[];
  int* rowinfo = reinterpret_cast<int*>(lds + a.lds_floats);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = logical / a.G;
  const int g = logical - tile * a.G;
  const int I0 = tile * (64 * K);
  const int t0 = I0 / a.Pp;
  build_row_table(a, t0, rowinfo);

  float acc[OCW][K];
#pragma unroll
  for (int o = 0; o < OCW; o++)
#pragma unroll
    for (int b = 0; b < K; b++) acc[o][b] = 0.0f;

  const float* lane_lds = lds + (I0 - t0 * a.Pp) + lane;
  const int slot0 = (g * kWaves + wave) * OCW;

  for (int k = 0; k < a.nch; k++) {
    const int c0 = k * a.Cc;
    const int cc = min(a.Cc, a.C - c0);
    __syncthreads();  // row table ready / previous chunk fully consumed
    stage_chunk(a, x, rowinfo, lds, c0, cc);
    __syncthreads();
#pragma unroll
    for (int o = 0; o < OCW; o++) {
      const int2 sg = seg[(slot0 + o) * a.nch + k];
      int j = sg.x;
      for (; j + 8 <= sg.y; j += 8) {
        uint2 e[8];
#pragma unroll
        for (int u = 0; u < 8; u++) e[u] = ent[j + u];
#pragma unroll
        for (int u = 0; u < 8; u++) fma_entry<K>(acc[o], lane_lds, e[u]);
      }
      for (; j < sg.y; j++) fma_entry<K>(acc[o], lane_lds, ent[j]);
    }
  }

  int ob[K];
  output_bases<K>(a, I0, lane, ob);
  const int plane = a.E * a.F;
#pragma unroll
  for (int o = 0; o < OCW; o++) {
    const int row = slot_row[slot0 + o];
    if (row < 0) continue;
#pragma unroll
    for (int b = 0; b < K; b++)
      if (ob[b] >= 0) __builtin_nontemporal_store(acc[o][b], y + ob[b] + row * plane);
  }
}

// Dense direct baseline: identical tiling and staging, every tap (c, r, s) of every
// output channel, weights read wave-uniformly from the dense M*C*R*S tensor.  Output
// channels are dealt out contiguously: slot (g, wave, o) -> channel (g*8 + wave)*OCW + o.
template <int K, int OCW>
__global__ __launch_bounds__(kThreads) void dense_direct_fwd(
    const KArgs a, const float* __restrict__ x, float* __restrict__ y,
    const float* __restrict__ wd) {
  extern __shared__ float lds[];
  int* rowinfo = reinterpret_cast<int*>(lds + a.lds_floats);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = logical / a.G;
  const int g = logical - tile * a.G;
  const int I0 = tile * (64 * K);
  const int t0 = I0 / a.Pp;
  build_row_table(a, t0, rowinfo);

  float acc[OCW][K];
#pragma unroll
  for (int o = 0; o < OCW; o++)
#pragma unroll
    for (int b = 0; b < K; b++) acc[o][b] = 0.0f;

  const float* lane_lds = lds + (I0 - t0 * a.Pp) + lane;
  const int slot0 = (g * kWaves + wave) * OCW;
  const int RS = a.R * a.S;

  for (int k = 0; k < a.nch; k++) {
    const int c0 = k * a.Cc;
    const int cc = min(a.Cc, a.C - c0);
    __syncthreads();
    stage_chunk(a, x, rowinfo, lds, c0, cc);
    __syncthreads();
#pragma unroll
    for (int o = 0; o < OCW; o++) {
      const int row = slot0 + o;
      if (row >= a.M) continue;
      const float* wr = wd + ((long long)row * a.C + c0) * RS;
      for (int cl = 0; cl < cc; cl++) {
        int rq = 0, rm = 0;
        for (int r = 0; r < a.R; r++) {
          int sq = 0, sm = 0;
          for (int s = 0; s < a.S; s++) {
            const int off = cl * a.CHS + (rm * a.st + sm) * a.PH + rq * a.Pp + sq;
            const float w = wr[(cl * a.R + r) * a.S + s];
            const float* p = lane_lds + off;
#pragma unroll
            for (int b = 0; b < K; b++) acc[o][b] = fmaf(w, p[64 * b], acc[o][b]);
            if (++sm == a.st) { sm = 0; sq++; }
          }
          if (++rm == a.st) { rm = 0; rq++; }
        }
      }
    }
  }

  int ob[K];
  output_bases<K>(a, I0, lane, ob);
  const int plane = a.E * a.F;
#pragma unroll
  for (int o = 0; o < OCW; o++) {
    const int row = slot0 + o;
    if (row >= a.M) continue;
#pragma unroll
    for (int b = 0; b < K; b++)
      if (ob[b] >= 0) __builtin_nontemporal_store(acc[o][b], y + ob[b] + row * plane);
  }
}

using SparseFn = void (*)(KArgs, const float*, float*, const uint2*, const int2*, const int*);
using DenseFn = void (*)(KArgs, const float*, float*, const float*);

#define SC_FOR_EACH_PLAN(X) \
  X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(1, 16) \
  X(2, 1) X(2, 2) X(2, 4) X(2, 8) X(2, 16) \
  X(4, 1) X(4, 2) X(4, 4) X(4, 8) X(4, 16) \
  X(8, 1) X(8, 2) X(8, 4) X(8, 8) X(8, 16)

static SparseFn pick_sparse(int K, int OCW) {
#define SC_CASE(KK, OO) if (K == KK && OCW == OO) return sparse_direct_fwd<KK, OO>;
  SC_FOR_EACH_PLAN(SC_CASE)
#undef SC_CASE
  return nullptr;
}

static DenseFn pick_dense(int K, int OCW) {
#define SC_CASE(KK, OO) if (K == KK && OCW == OO) return dense_direct_fwd<KK, OO>;
  SC_FOR_EACH_PLAN(SC_CASE)
#undef SC_CASE
  return nullptr;
}

static hipError_t allow_lds(const void* fn, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks) {
  SparseFn fn = pick_sparse(p.K, p.OCW);
  if (!fn) return (int)hipErrorInvalidDeviceFunction;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), p.lds_bytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fn, dim3(nblocks), dim3(kThreads), p.lds_bytes, reinterpret_cast<hipStream_t>(stream), a,
                     a.x, a.y, reinterpret_cast<const uint2*>(a.ent), reinterpret_cast<const int2*>(a.seg),
                     a.slot_row);
  return (int)hipGetLastError();
}

int launch_dense(const Plan& p, const KArgs& a, void* stream, int nblocks) {
  DenseFn fn = pick_dense(p.K, p.OCW);
  if (!fn) return (int)hipErrorInvalidDeviceFunction;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), p.lds_bytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fn, dim3(nblocks), dim3(kThreads), p.lds_bytes, reinterpret_cast<hipStream_t>(stream), a,
                     a.x, a.y, a.wd);
  return (int)hipGetLastError();
}

}  // namespace sc
