// gfx950 kernels of the second mapping: "Escoin: Efficient Sparse Convolutional Neural
// Network Inference on GPUs", dataflow and data-placement sections (its Fig. 6 thread
// mapping and its pad_in step).
//
//   pad_in - copies the NCHW input into a zero-padded NCHW buffer (planes of
//            (H + 2 pad) x (W + 2 pad)), so that the convolution needs no bounds checks;
//   sconv  - one output channel per workgroup (weight stationary): the workgroup copies its
//            CSR row {stretched offset against the padded pitch, value} into LDS, and each
//            thread accumulates P output positions of one image in registers, P * 256
//            consecutive positions per workgroup.  For every non-zero, the weight is read
//            from LDS (one broadcast read per wavefront), the inputs come from the padded
//            buffer through the caches (consecutive lanes read consecutive words for
//            stride 1), and each lane does P FMAs.  Workgroups of all output channels of one
//            spatial tile run next to each other on one XCD, so they share the tile's input in
//            that XCD's L2 cache.
//
// Unlike the LDS-tile kernel (kernels.hip), nothing here stages the input: every non-zero
// re-reads its input words through L1/L2.  The two are kept side by side to measure that
// choice on this chip.
#include <hip/hip_runtime.h>

#include <mutex>

#include "plan.h"
#include "xcd.h"

namespace sc {

namespace {

// Static workspace for callers that cannot allocate (sparseconv_forward_noalloc): device
// memory of this code object, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): it uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// One thread per padded word; a workgroup covers a run of one padded plane.
__global__ __launch_bounds__(256) void pad_in(const float* __restrict__ x, float* __restrict__ xp, int H, int W,
                                              int pad, int Hp, int Wp, int runs_per_plane) {
  const int plane = blockIdx.x / runs_per_plane;  // n * C + c
  const int i = (blockIdx.x - plane * runs_per_plane) * 256 + threadIdx.x;
  if (i >= Hp * Wp) return;
  const int yp = i / Wp, xq = i - yp * Wp;
  const int iy = yp - pad, ix = xq - pad;
  float v = 0.0f;
  if (iy >= 0 && iy < H && ix >= 0 && ix < W) v = x[(long long)plane * H * W + (long long)iy * W + ix];
  xp[(long long)plane * Hp * Wp + i] = v;
}

// Raw buffer resource over [base, base + nbytes) (gfx9 family dword format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// One fp32 word at byte offset voff + soff of the buffer (the builtin returns the raw bits).
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff, soff, 0));
}

template <int P>
__global__ __launch_bounds__(256) void sconv(const EscoinArgs a, const float* __restrict__ xp,
                                             float* __restrict__ y, const uint2* __restrict__ ent,
                                             const int* __restrict__ rowptr) {
  extern __shared__ uint2 wrow[];
  const int t = threadIdx.x;
  // block -> (output channel m fastest, then spatial tile, then image); consecutive ids on
  // one XCD, so that the workgroups of a tile's output channels share that XCD's L2
  const int b = xcd_logical(blockIdx.x, gridDim.x);
  const int m = b % a.M;
  const int rest = b / a.M;
  const int tile = rest % a.tiles;
  const int n = rest / a.tiles;
  const int EF = a.E * a.F;
  // P output positions of this thread, 256 apart; a position past the plane reads word 0 of
  // the image (in range) and is not stored
  int q[P];
  uint32_t vb[P];  // byte offset of the position's first tap within the image's padded planes
#pragma unroll
  for (int p = 0; p < P; p++) {
    q[p] = tile * (256 * P) + p * 256 + t;
    const int qq = q[p] < EF ? q[p] : 0;
    const int e = qq / a.F, f = qq - e * a.F;
    vb[p] = 4u * (uint32_t)(e * a.st * a.Wp + f * a.st);
  }
  const float* img = xp + (long long)n * a.img_words;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(img, 4u * (uint32_t)a.img_words);
  float acc[P];
#pragma unroll
  for (int p = 0; p < P; p++) acc[p] = 0.0f;
  const int j0 = rowptr[m], j1 = rowptr[m + 1];
  for (int c0 = j0; c0 < j1; c0 += a.chunk) {
    const int cn = min(a.chunk, j1 - c0);
    __syncthreads();  // the previous chunk's reads are done
    for (int i = t; i < cn; i += 256) wrow[i] = ent[c0 + i];
    __syncthreads();
    // four non-zeros at a time: 4 * P loads in flight per wavefront before the FMAs
    int j = 0;
    for (; j + 4 <= cn; j += 4) {
      float v[4][P], w[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const uint2 e = wrow[j + u];
        const int so = __builtin_amdgcn_readfirstlane((int)(4u * e.x));
        w[u] = __uint_as_float(e.y);
#pragma unroll
        for (int p = 0; p < P; p++) v[u][p] = load_f32(rs, vb[p], so);
      }
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int p = 0; p < P; p++) acc[p] = fmaf(w[u], v[u][p], acc[p]);
    }
    for (; j < cn; j++) {
      const uint2 e = wrow[j];
      const int so = __builtin_amdgcn_readfirstlane((int)(4u * e.x));
      const float w = __uint_as_float(e.y);
#pragma unroll
      for (int p = 0; p < P; p++) acc[p] = fmaf(w, load_f32(rs, vb[p], so), acc[p]);
    }
  }
  float* yo = y + ((long long)n * a.M + m) * EF;
#pragma unroll
  for (int p = 0; p < P; p++)
    if (q[p] < EF) yo[q[p]] = acc[p];
}

}  // namespace

int scratch_address(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return (int)hipSuccess;
}

int launch_escoin(const EscoinArgs& a, const float* x, float* xp, float* y, const uint32_t* ent,
                  const int32_t* rowptr, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int runs = (a.Hp * a.Wp + 255) / 256;
  hipLaunchKernelGGL(pad_in, dim3((unsigned)(a.N * a.C * runs)), dim3(256), 0, s, x, xp, a.H, a.W, a.pad, a.Hp,
                     a.Wp, runs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  const long long blocks = (long long)a.M * a.tiles * a.N;
  hipLaunchKernelGGL(sconv<kEscoinP>, dim3((unsigned)blocks), dim3(256), a.chunk * 8, s, a, xp, y,
                     reinterpret_cast<const uint2*>(ent), rowptr);
  return (int)hipGetLastError();
}

}  // namespace sc
