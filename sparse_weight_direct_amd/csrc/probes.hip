// Roof probes timed by the benchmark next to the copy reference: small kernels that measure
// what the chip delivers to the instruction mixes the convolution kernels are made of.
//
//   scprobe_fma   - wavefronts issuing independent v_fmac_f32 with a 32-bit literal weight
//                   (the weights-in-code kernels' instruction) or a VGPR weight, registers
//                   only: the fp32 FMA rate of the vector ALUs for a given number of wavefronts
//                   per SIMD;
//   scprobe_lds   - wavefronts issuing ds_read_b32 or ds_read_b128 from LDS into registers:
//                   the LDS read bandwidth;
//   scprobe_read  - a grid-stride stream of 16-byte loads: the HBM read rate of pure reads.
//
// Each lane writes one float at the end (so nothing is optimised away) to out[global id]; the
// caller sizes out for blocks * 256 floats.
#include <hip/hip_runtime.h>

namespace {

#define SC_REP2(x) x x
#define SC_REP8(x) SC_REP2(SC_REP2(SC_REP2(x)))
#define SC_REP64(x) SC_REP8(SC_REP8(x))
#define SC_FMA8_LIT                                                                                  \
  "v_fmac_f32 %0, 0x3f800001, %8\n v_fmac_f32 %1, 0x3f800002, %8\n v_fmac_f32 %2, 0x3f800003, %8\n" \
  " v_fmac_f32 %3, 0x3f800004, %8\n v_fmac_f32 %4, 0x3f800005, %8\n v_fmac_f32 %5, 0x3f800006, %8\n" \
  " v_fmac_f32 %6, 0x3f800007, %8\n v_fmac_f32 %7, 0x3f800008, %8\n"
#define SC_FMA8_VGPR                                                                                  \
  "v_fmac_f32 %0, %9, %8\n v_fmac_f32 %1, %9, %8\n v_fmac_f32 %2, %9, %8\n v_fmac_f32 %3, %9, %8\n" \
  " v_fmac_f32 %4, %9, %8\n v_fmac_f32 %5, %9, %8\n v_fmac_f32 %6, %9, %8\n v_fmac_f32 %7, %9, %8\n"

// 512 FMAs per iteration and wavefront, 8 independent accumulators
template <bool LIT>
__global__ __launch_bounds__(256) void fma_probe(float* out, float seed, int iters) {
  float a0 = seed, a1 = seed, a2 = seed, a3 = seed, a4 = seed, a5 = seed, a6 = seed, a7 = seed;
  const float x = seed * 0.5f, w = seed * 0.25f;
  for (int it = 0; it < iters; it++) {
    if (LIT)
      asm volatile(SC_REP64(SC_FMA8_LIT)
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "v"(x));
    else
      asm volatile(SC_REP64(SC_FMA8_VGPR)
                   : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                   : "v"(x), "v"(w));
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

// 64 reads per iteration and wavefront (8 in flight at a time) from a 16 KB LDS array filled
// by the workgroup; each lane reads consecutive words (b32: 256 bytes per wavefront read,
// b128: 1 KB), without bank conflicts; the values are summed so the reads cannot be dropped
constexpr int kLdsBytes = 16384;
typedef float f4 __attribute__((ext_vector_type(4)));

template <int WORDS>
__global__ __launch_bounds__(256) void lds_probe(float* out, int iters) {
  __shared__ float buf[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x) buf[i] = (float)i;
  __syncthreads();
  // byte address of the lane's first word: the lanes of a wavefront read consecutive words;
  // every read stays inside buf (b32: at most 1020 + 7168 + 4 bytes, b128: at most
  // 4080 + 10752 + 16 bytes, both below kLdsBytes)
  const unsigned base = (unsigned)threadIdx.x * 4u * WORDS;
  float acc = 0.0f;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if (WORDS == 1) {
        float v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b32 %0, %8\n ds_read_b32 %1, %8 offset:1024\n ds_read_b32 %2, %8 offset:2048\n"
            " ds_read_b32 %3, %8 offset:3072\n ds_read_b32 %4, %8 offset:4096\n ds_read_b32 %5, %8 offset:5120\n"
            " ds_read_b32 %6, %8 offset:6144\n ds_read_b32 %7, %8 offset:7168\n s_waitcnt lgkmcnt(0)"
            : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
            : "v"(base));
        acc += v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
      } else {
        f4 v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:1536\n ds_read_b128 %2, %8 offset:3072\n"
            " ds_read_b128 %3, %8 offset:4608\n ds_read_b128 %4, %8 offset:6144\n ds_read_b128 %5, %8 offset:7680\n"
            " ds_read_b128 %6, %8 offset:9216\n ds_read_b128 %7, %8 offset:10752\n s_waitcnt lgkmcnt(0)"
            : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
            : "v"(base));
        acc += v0.x + v1.y + v2.z + v3.w + v4.x + v5.y + v6.z + v7.w;
      }
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Streams n4 16-byte vectors through the vector memory path (each thread 4 loads in flight per
// step of a grid-stride loop) and writes one value per thread: the HBM read rate of a pure
// read stream.
__global__ __launch_bounds__(256) void read_probe(const f4* __restrict__ x, long long n4, float* out) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const f4 a = x[i], b = x[i + stride], c = x[i + 2 * stride], d = x[i + 3 * stride];
    acc += a + b + c + d;
  }
  for (; i < n4; i += stride) acc += x[i];
  out[(long long)blockIdx.x * blockDim.x + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

}  // namespace

extern "C" {

// Reads n4 16-byte vectors at x with blocks workgroups of 256 threads; out holds blocks * 256
// floats.  Returns a hipError_t.
int scprobe_read(const void* x, long long n4, float* out, int blocks, void* stream) {
  if (!x || !out || n4 < 1 || blocks < 1) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(read_probe, dim3(blocks), dim3(256), 0, s, static_cast<const f4*>(x), n4, out);
  return (int)hipGetLastError();
}

// kind 0: literal-weight FMAs, 1: VGPR-weight FMAs.  blocks workgroups of 256 threads (4
// wavefronts; one per SIMD of a CU), iters * 512 FMAs per wavefront.  Returns a hipError_t.
int scprobe_fma(float* out, int kind, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(fma_probe<true>, dim3(blocks), dim3(256), 0, s, out, 1.0f, iters);
  else
    hipLaunchKernelGGL(fma_probe<false>, dim3(blocks), dim3(256), 0, s, out, 1.0f, iters);
  return (int)hipGetLastError();
}

// words 1: ds_read_b32, 4: ds_read_b128.  blocks workgroups of 256 threads, iters * 64 reads
// per wavefront (8 in flight).  Returns a hipError_t.
int scprobe_lds(float* out, int words, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (words != 1 && words != 4)) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (words == 1)
    hipLaunchKernelGGL(lds_probe<1>, dim3(blocks), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(lds_probe<4>, dim3(blocks), dim3(256), 0, s, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
