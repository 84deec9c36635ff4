// gfx950 dense direct convolution: the on-GPU dense baseline (sparseconv_dense_forward).  Every
// filter tap, zeros included, of a dense M x C x R x S weight tensor that already sits on the
// device: the dense work of Tuteja et al., "Theoretical and Empirical Analysis of Sparse
// Convolution", Sec. 4 Eq. (5), against which their Sec. 6.1 / Fig. 5 measure the sparse kernel.
//
// A wavefront holds K output positions per lane (K tiles of 64 consecutive positions in NCHW
// output order, lane = position within a tile) and the accumulators of MG output channels:
// K*MG VGPRs for the whole input.  It walks the filter rows r, then the input channels c,
// then the filter columns s.  Per filter row it computes, for every position and column, the
// offset of X[n, 0, e*st - pad + r, f*st - pad + s] (the out-of-range marker 0x80000000 in
// the padding, so the bounded buffer load returns 0); per channel only the scalar offset
// c*H*W*4 changes.  Per (r, c) it loads K*S row vectors and adds W[m, c, r, s] times them to
// the accumulators: K*MG*S FMAs with the weight as a scalar operand.  The weight address
// depends only on the wavefront's channel group and the loop counters, so the weights arrive
// through scalar loads straight from the caller's M x C x R x S array.
//
// Work units are (tile group, channel group); the channel group runs fastest, so the
// wavefronts of a workgroup read the same input rows (through L1), and consecutive workgroups
// sit on one XCD (shared L2 for the halo rows of neighbouring tiles).
#include <hip/hip_runtime.h>

#include "plan.h"
#include "xcd.h"

namespace sc {

namespace {

constexpr int kWaves = 4;         // wavefronts per workgroup
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// SW: filter columns per pass (the filter row is walked in passes of SW columns; GUARD: the
// last pass is partial).  K: positions per lane.  MG: output channels per wavefront.
template <int SW, bool GUARD, int K, int MG>
__global__ __launch_bounds__(64 * kWaves) void dense_direct_fwd(const float* __restrict__ w,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ y, const DenseArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = xcd_logical(blockIdx.x, gridDim.x) * kWaves + wave;
  if (unit >= a.tgroups * a.groups) return;
  const int tg = unit / a.groups;
  const int m0 = (unit - tg * a.groups) * MG;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x), (short)0, a.x_bytes,
                                                                      0x00020000);
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(y, (short)0, a.y_bytes, 0x00020000);
  // per position: image base (words), first input row and column of its window, validity
  int img[K], iy0[K], ix0[K];
  bool valid[K];
  uint32_t obase[K];
#pragma unroll
  for (int k = 0; k < K; k++) {
    const int q = (tg * K + k) * 64 + lane;
    valid[k] = q < a.qtot;
    const int n = valid[k] ? q / a.EF : 0;
    const int rem = valid[k] ? q - n * a.EF : 0;
    const int e = rem / a.F, f = rem - e * a.F;
    img[k] = n * a.CHW;
    iy0[k] = e * a.st - a.pad;
    ix0[k] = f * a.st - a.pad;
    obase[k] = valid[k] ? 4u * (uint32_t)(n * a.MEF + rem) : kOob;
  }
  float acc[MG][K];
#pragma unroll
  for (int m = 0; m < MG; m++)
#pragma unroll
    for (int k = 0; k < K; k++) acc[m][k] = 0.0f;
  // a partial last group computes channel M - 1 in its surplus slots and never stores them
  const int mlast = a.M - 1 - m0;
  const float* __restrict__ wm0 = w + (long long)m0 * a.CRS;
  for (int r = 0; r < a.R; r++) {
    for (int s0 = 0; s0 < a.S; s0 += SW) {
      uint32_t voff[SW][K];
#pragma unroll
      for (int k = 0; k < K; k++) {
        const int iy = iy0[k] + r;
        const bool row_ok = valid[k] && iy >= 0 && iy < a.H;
#pragma unroll
        for (int j = 0; j < SW; j++) {
          const int ix = ix0[k] + s0 + j;
          const bool ok = row_ok && ix >= 0 && ix < a.W && (!GUARD || s0 + j < a.S);
          voff[j][k] = ok ? 4u * (uint32_t)(img[k] + iy * a.W + ix) : kOob;
        }
      }
      // W[m0 + m, c, r, s0 + j] is wm0[m*CRS + c*RS + r*S + s0 + j]
      uint32_t soff = 0;
      int wo = r * a.S + s0;
      for (int c = 0; c < a.C; c++, soff += a.HW4, wo += a.RS) {
        float win[SW][K];
#pragma unroll
        for (int j = 0; j < SW; j++)
#pragma unroll
          for (int k = 0; k < K; k++) win[j][k] = bload(xr, voff[j][k], soff);
        // every weight of the step first (scalar loads in flight together), then the FMAs
        float wv[MG][SW];
#pragma unroll
        for (int m = 0; m < MG; m++) {
          const int wi = __builtin_amdgcn_readfirstlane(wo + min(m, mlast) * a.CRS);
#pragma unroll
          for (int j = 0; j < SW; j++) wv[m][j] = (GUARD && s0 + j >= a.S) ? 0.0f : wm0[wi + j];
        }
#pragma unroll
        for (int m = 0; m < MG; m++)
#pragma unroll
          for (int j = 0; j < SW; j++) {
            if (GUARD && s0 + j >= a.S) continue;
#pragma unroll
            for (int k = 0; k < K; k++) acc[m][k] = fmaf(wv[m][j], win[j][k], acc[m][k]);
          }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MG; m++) {
    if (m > mlast) break;
    const uint32_t so = 4u * (uint32_t)((m0 + m) * a.EF);
#pragma unroll
    for (int k = 0; k < K; k++)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, acc[m][k]), yr, obase[k], so, 0);
  }
}

template <int SW, bool GUARD, int K, int MG>
int launch_one(const DenseArgs& a, const float* w, const float* x, float* y, hipStream_t st, unsigned blocks) {
  hipLaunchKernelGGL((dense_direct_fwd<SW, GUARD, K, MG>), dim3(blocks), dim3(64 * kWaves), 0, st, w, x, y, a);
  return (int)hipGetLastError();
}

// Column passes of at most 3 (MG * SW weights held in scalar registers); a partial last pass
// skips its surplus columns.
template <int K, int MG>
int launch_shape(DenseArgs a, const float* w, const float* x, float* y, hipStream_t st) {
  a.tgroups = (int)((a.qtot + 64LL * K - 1) / (64LL * K));
  a.groups = (a.M + MG - 1) / MG;
  const long long units = (long long)a.tgroups * a.groups;
  if (units + kWaves >= (1LL << 31)) return (int)hipErrorInvalidConfiguration;
  const unsigned b = (unsigned)((units + kWaves - 1) / kWaves);
  switch (a.S) {
    case 1: return launch_one<1, false, K, MG>(a, w, x, y, st, b);
    case 2: return launch_one<2, false, K, MG>(a, w, x, y, st, b);
    case 4: return launch_one<2, false, K, MG>(a, w, x, y, st, b);
    default:
      return a.S % 3 == 0 ? launch_one<3, false, K, MG>(a, w, x, y, st, b)
                          : launch_one<3, true, K, MG>(a, w, x, y, st, b);
  }
}

struct Shape {
  int K, MG;
};
// Tile shapes, most work per wavefront first.  With one filter column per pass the scalar
// weight loads and their address arithmetic are paid per K FMAs, so S = 1 prefers fewer
// channels and more positions per wavefront.
constexpr Shape kShapesS1[] = {{4, 4}, {2, 4}};
constexpr Shape kShapes[] = {{3, 8}, {2, 8}, {2, 4}};

long long shape_waves(const DenseArgs& a, Shape s) {
  return (a.qtot + 64LL * s.K - 1) / (64LL * s.K) * ((a.M + s.MG - 1) / s.MG);
}

}  // namespace

// The first shape (in preference order) that gives every SIMD of the chip 1.5 wavefronts,
// else the one with the most wavefronts.
void dense_pick(const DenseArgs& a, int simds, int* K, int* MG) {
  const Shape* list = a.S == 1 ? kShapesS1 : kShapes;
  const int n = a.S == 1 ? 2 : 3;
  Shape best = list[0];
  for (int i = 0; i < n; i++) {
    if (2 * shape_waves(a, list[i]) >= 3LL * simds) {
      *K = list[i].K, *MG = list[i].MG;
      return;
    }
    if (shape_waves(a, list[i]) > shape_waves(a, best)) best = list[i];
  }
  *K = best.K, *MG = best.MG;
}

int launch_dense(DenseArgs a, const float* w, const float* x, float* y, int simds, void* stream) {
  int K = 0, MG = 0;
  dense_pick(a, simds, &K, &MG);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (K == 4 && MG == 4) return launch_shape<4, 4>(a, w, x, y, st);
  if (K == 3 && MG == 8) return launch_shape<3, 8>(a, w, x, y, st);
  if (K == 2 && MG == 8) return launch_shape<2, 8>(a, w, x, y, st);
  return launch_shape<2, 4>(a, w, x, y, st);
}

}  // namespace sc
