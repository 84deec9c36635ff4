// gfx950 kernel: sparse direct convolution (the dense direct baseline is the same kernel
// on a handle that stores every filter tap).
//
// Work decomposition.  A tile is 64*K consecutive extended output positions (plan.h); a
// work unit is one tile for one group of output channels.  The grid is persistent: every
// CU runs the workgroups its LDS and registers allow, and each workgroup owns one
// contiguous run of units (runs differ by at most one unit), so neighbouring tiles, whose
// staged rows overlap, are handled by the same workgroup one after the other.
//
// Per workgroup (NW wavefronts), the units are walked as a stream of steps
// (unit, chunk of Cc input channels):
//   staging  - each step's input rows (stride-phase planes, zero padding included) are
//              copied HBM -> LDS by direct buffer loads into LDS (gfx950 LDS DMA) into
//              one of two ring slots while the other is consumed.  A wavefront owns
//              fixed 64-word blocks of the staged channel layout; a block's per-lane
//              source offsets are computed once per step and serve every channel of the
//              chunk (only a scalar offset of c*H*W words changes), and padding words
//              get an out-of-range offset, which the load turns into 0;
//   compute  - each wavefront walks the non-zeros of its output-channel slots for the
//              step.  Its block of {enc, value} non-zeros is staged into the same ring slot
//              by the same loads; the wavefront reads it 64 entries at a time (one per
//              lane) and broadcasts each entry with v_readlane.  Per non-zero each lane
//              does one address add, K LDS reads 64 words apart and K fp32 FMAs;
//   store    - after a unit's last chunk, coalesced NCHW stores of the valid positions;
//              slots of channels without non-zeros store exact zeros.
// One barrier per step: before it, each wavefront waits (vmcnt) until its own loads of the
// step have landed; after it, the slot consumed in the previous step is refilled with the
// next step while this one is computed (two ring slots).
//
// Prior art kept from the pages: the input tile plus halo staged once per block and reused
// by every output channel, the packed per-non-zero word, and per-thread register
// accumulators (Tuteja et al., Sec. 5.1-5.5); the wave-uniform weight with lanes over
// consecutive output positions (the thread-per-output dataflow of "Escoin").
#include <hip/hip_runtime.h>

#include "plan.h"

namespace sc {

constexpr uint32_t kOutOfRange = 0x80000000u;  // >= every buffer's num_records: loads 0

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer resource: base, no stride, num_records bytes, dword data format (gfx9 family).
// Arguments are wave-uniform; readfirstlane moves values read from LDS into scalar registers.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t nbytes) {
  const unsigned long long b = (unsigned long long)base;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
  r.w = 0x00020000;
  return r;
}

// One direct global->LDS load (LDS DMA): lane i writes the dword at byte voff + soff of the
// buffer (0 when out of range) to LDS byte address lds + 4*i.  Padding lanes carry
// voff = 0x80000000, beyond num_records (< 2^31) with or without soff (< 2^31), so the
// zero does not depend on whether the range check includes the scalar offset.  Issued
// from inline asm so the compiler does not treat it as an LDS store it must wait for
// before every LDS read; completion is awaited explicitly (vmcnt) at the step barrier.
__device__ __forceinline__ void lds_dma_dword(v4i rsrc, const float* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc), "s"(so)
      : "memory", "m0");
}

// Workgroups are handed to the 8 XCDs round-robin; renumber them so that consecutive
// logical ids (hence adjacent runs of tiles, which share halo rows) sit on one XCD's L2.
__device__ __forceinline__ int xcd_logical(int b, int nb) {
  const int q = nb >> 3, rmd = nb & 7;
  const int xcd = b & 7, k = b >> 3;
  return xcd < rmd ? xcd * (q + 1) + k : rmd * (q + 1) + (xcd - rmd) * q + k;
}

// Wait until this wavefront's staging loads have landed, then barrier.  The empty asm keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0); expcnt, lgkmcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row table of a tile, per wavefront: entry py*NRmax + j holds the word offset of the
// input row behind phase row j of phase row-plane py, relative to channel 0 of the tile's
// first image n0 (returned): (n-n0)*C*H*W + y*W, or -1 for padding rows and rows past the
// last image.
__device__ __forceinline__ int tile_rows(const KArgs& a, int tile, int K, int lane, int* rowtab) {
  const int t0 = tile * (64 * K) / a.Pp;
  const int n0 = t0 / a.HYp;
  for (int i = lane; i < a.st * a.NRmax; i += 64) {
    const int py = i / a.NRmax;
    const int j = i - py * a.NRmax;
    const int Tr = t0 + j;
    const int n = Tr / a.HYp;
    const int y = (Tr - n * a.HYp) * a.st + py - a.pad;
    rowtab[i] = (n < a.N && y >= 0 && y < a.H) ? ((n - n0) * a.C * a.H + y) * a.W : -1;
  }
  return n0;
}

// Source byte offset of the lane's word in block blk of the staged channel layout
// (channel term excluded), or out of range for padding, missing rows and the slack at the
// end of a channel.
__device__ __forceinline__ uint32_t block_voff(const KArgs& a, int blk, int lane, const int* rowtab) {
  const int w = 64 * blk + lane;
  const int ph = w / a.PH;
  uint32_t off = kOutOfRange;
  if (ph < a.st * a.st) {
    const int rem = w - ph * a.PH;
    const int j = rem / a.Pp;
    const int xq = rem - j * a.Pp;
    const int py = ph / a.st;
    const int xg = xq * a.st + (ph - py * a.st) - a.pad;
    if (xg >= 0 && xg < a.W) {
      const int r = rowtab[py * a.NRmax + j];
      if (r >= 0) off = 4u * (uint32_t)(r + xg);
    }
  }
  return off;
}

// Start the asynchronous copy of channels [c0, c0 + ncl) of a tile into the input part of a
// ring slot: the wavefront's blocks blk = wave, wave + NW, ... of every channel.
template <int NW>
__device__ __forceinline__ void stage_rows(const KArgs& a, v4i rsrc, int c0, int ncl, float* slot, int wave,
                                           int lane, const int* rowtab) {
  for (int blk = wave; blk < a.nblk; blk += NW) {
    const uint32_t voff = block_voff(a, blk, lane, rowtab);
    uint32_t soff = 4u * (uint32_t)(c0 * a.HW);
    const float* dst = slot + 64 * blk;
    for (int cl = 0; cl < ncl; cl++) {
      lds_dma_dword(rsrc, dst, voff, soff);
      dst += a.CHS;
      soff += 4u * (uint32_t)a.HW;
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
__device__ __forceinline__ void fma_entry(float (&acc)[K], const float* lane_lds, uint32_t off, float w) {
  const float* p = lane_lds + off;
#pragma unroll
  for (int b = 0; b < K; b++) acc[b] = fmaf(w, p[64 * b], acc[b]);
}

// np pairs of consecutive non-zeros starting at lane r (even) of a group of 64 entries
// held one per lane: each entry is broadcast to the wave with v_readlane (no scalar memory
// access in the loop).  The empty asm after the reads keeps the scheduler from
// interleaving each read with its FMAs (under register pressure it otherwise waits on
// every read); a pair keeps 2*K LDS reads in flight.
template <int K>
__device__ __forceinline__ void pair(float (&acc)[K], const float* lane_lds, const uint2 grp, int l) {
  const uint32_t o0 = (uint32_t)__builtin_amdgcn_readlane((int)grp.x, l);
  const uint32_t o1 = (uint32_t)__builtin_amdgcn_readlane((int)grp.x, l + 1);
  const float w0 = __int_as_float(__builtin_amdgcn_readlane((int)grp.y, l));
  const float w1 = __int_as_float(__builtin_amdgcn_readlane((int)grp.y, l + 1));
  const float* p0 = lane_lds + o0;
  const float* p1 = lane_lds + o1;
  float v0[K], v1[K];
#pragma unroll
  for (int b = 0; b < K; b++) v0[b] = p0[64 * b];
#pragma unroll
  for (int b = 0; b < K; b++) v1[b] = p1[64 * b];
  asm volatile("" ::: "memory");
#pragma unroll
  for (int b = 0; b < K; b++) acc[b] = fmaf(w0, v0[b], acc[b]);
#pragma unroll
  for (int b = 0; b < K; b++) acc[b] = fmaf(w1, v1[b], acc[b]);
}

template <int K>
__device__ __forceinline__ void run_pairs(float (&acc)[K], const float* lane_lds, const uint2 grp, int l, int np) {
  const int lend = l + 2 * np;
  if (np & 1) {
    pair<K>(acc, lane_lds, grp, l);
    l += 2;
  }
  for (; l < lend; l += 4) {
    pair<K>(acc, lane_lds, grp, l);
    pair<K>(acc, lane_lds, grp, l + 2);
  }
}

// Stage the wavefront's block of non-zeros (stream entries [b0, b1)) into its share of a
// ring slot: QE loads of 64 words (32 entries) each; words past the block's end load as 0.
// Entry e of the block lands at word nin + T*(e/32) + 64*wave + 2*(e%32) of the slot.
template <int T>
__device__ __forceinline__ void stage_block(const KArgs& a, const uint2* __restrict__ ent, int b0, int b1,
                                            float* slot, int wave, int lane) {
  const v4i rsrc = make_rsrc(ent + b0, (uint32_t)(b1 - b0) * 8u);
  for (int q = 0; q < a.QE; q++) lds_dma_dword(rsrc, slot + a.nin + T * q + 64 * wave, 4u * (64 * q + lane), 0u);
}

// One step: the wavefront's slots and their non-zeros of this chunk, read from the block
// staged in the ring slot: header entries {count of slot o, 0} (OCW of them, rounded up to
// an even number), then the slots' non-zeros {enc, value} in slot order, each slot's run
// padded to an even length with zero-weight entries so that it is walked in pairs that
// never straddle a group of 64 (lane i holds entry i of the group).
template <int K, int OCW, int NW>
__device__ __forceinline__ void sparse_step(const KArgs& a, float (&acc)[OCW][K], const float* lane_lds,
                                            const float* slot, int wave, int lane) {
  constexpr int T = NW * 64;
  constexpr int HDR = (OCW + 1) & ~1;
  const uint32_t* eb = reinterpret_cast<const uint32_t*>(slot + a.nin) + 64 * wave;
  const int emax = 32 * a.QE - 1;
  auto group = [&](int base) -> uint2 {
    const int e = min(base + lane, emax);
    return *reinterpret_cast<const uint2*>(eb + T * (e >> 5) + 2 * (e & 31));
  };
  const uint2 head = group(0);
  uint2 cur = head;
  int r = HDR;   // next entry's lane within the current group
  int base = 0;  // entry index of the current group's lane 0
#pragma unroll
  for (int o = 0; o < OCW; o++) {
    int n = __builtin_amdgcn_readlane((int)head.x, o);  // even
    if (n == 0) continue;
    if (r + n <= 64) {  // the run lies in the current group
      run_pairs<K>(acc[o], lane_lds, cur, r, n >> 1);
      r += n;
      continue;
    }
    do {
      if (r == 64) {
        base += 64;
        cur = group(base);
        r = 0;
      }
      const int take = min(n, 64 - r);
      run_pairs<K>(acc[o], lane_lds, cur, r, take >> 1);
      r += take;
      n -= take;
    } while (n > 0);
  }
}

// Pointers are separate restrict-qualified arguments so the compiler knows the streams
// are read-only.
template <int K, int OCW, int NW>
__global__ __launch_bounds__(NW * 64, 4) void sparse_direct_fwd(
    const KArgs a, const float* __restrict__ x, float* __restrict__ y,
    const uint2* __restrict__ ent, const int* __restrict__ bstart,
    const int* __restrict__ slot_row) {
  constexpr int T = NW * 64;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int* rowtab = reinterpret_cast<int*>(lds + 2 * a.slot_words) + wave * a.rt;
  int* bst = reinterpret_cast<int*>(lds + 2 * a.slot_words) + NW * a.rt;

  const int b = xcd_logical(blockIdx.x, gridDim.x);
  const long long units = (long long)a.ntiles * a.G;
  const int u0 = (int)(units * b / gridDim.x);
  const int u1 = (int)(units * (b + 1) / gridDim.x);
  const int S = (u1 - u0) * a.nch;
  if (S == 0) return;

  for (int i = threadIdx.x; i < a.G * NW * (a.nch + 1); i += T) bst[i] = bstart[i];
  __syncthreads();

  // issue side: the next step to stage (unit = tile * G + g, chunk is_k, ring slot is_buf)
  int is_tile = u0 / a.G, is_g = u0 - (u0 / a.G) * a.G, is_k = 0, is_buf = 0, is_new_tile = 1;
  v4i rsrc = make_rsrc(x, 0u);
  auto issue = [&]() {
    if (is_new_tile) {
      const int n0 = tile_rows(a, is_tile, K, lane, rowtab);
      const long long first = (long long)n0 * a.C * a.HW;
      rsrc = make_rsrc(x + first, (uint32_t)min((a.x_words - first) * 4, 0x7ffffff0LL));
      is_new_tile = 0;
    }
    const int* bw = bst + (is_g * NW + wave) * (a.nch + 1) + is_k;
    float* slot = lds + is_buf * a.slot_words;
    stage_block<T>(a, ent, bw[0], bw[1], slot, wave, lane);
    const int c0 = is_k * a.Cc;
    stage_rows<NW>(a, rsrc, c0, min(a.Cc, a.C - c0), slot, wave, lane, rowtab);
    is_buf ^= 1;
    if (++is_k == a.nch) {
      is_k = 0;
      if (++is_g == a.G) {
        is_g = 0;
        is_tile++;
        is_new_tile = 1;
      }
    }
  };
  issue();

  float acc[OCW][K];
#pragma unroll
  for (int o = 0; o < OCW; o++)
#pragma unroll
    for (int q = 0; q < K; q++) acc[o][q] = 0.0f;

  int tile = u0 / a.G, g = u0 - (u0 / a.G) * a.G, ck = 0, cbuf = 0;
  int I0 = tile * (64 * K);
  int lane_pos = I0 - (I0 / a.Pp) * a.Pp + lane;
  for (int s = 0; s < S; s++) {
    step_barrier();  // step s landed; every wavefront is done with the other slot
    if (s + 1 < S) issue();
    const float* slot = lds + cbuf * a.slot_words;
    sparse_step<K, OCW, NW>(a, acc, slot + lane_pos, slot, wave, lane);
    cbuf ^= 1;
    if (++ck == a.nch) {
      int ob[K];
      output_bases<K>(a, I0, lane, ob);
      const int plane = a.E * a.F;
#pragma unroll
      for (int o = 0; o < OCW; o++) {
        const int row = slot_row[(g * NW + wave) * OCW + o];
        if (row >= 0) {
#pragma unroll
          for (int q = 0; q < K; q++)
            if (ob[q] >= 0) __builtin_nontemporal_store(acc[o][q], y + ob[q] + row * plane);
        }
#pragma unroll
        for (int q = 0; q < K; q++) acc[o][q] = 0.0f;
      }
      ck = 0;
      if (++g == a.G) {
        g = 0;
        tile++;
        I0 = tile * (64 * K);
        lane_pos = I0 - (I0 / a.Pp) * a.Pp + lane;
      }
    }
  }
}

using SparseFn = void (*)(KArgs, const float*, float*, const uint2*, const int*, const int*);

#define SC_FOR_EACH_KO(X, NW) \
  X(1, 1, NW) X(1, 2, NW) X(1, 4, NW) X(1, 8, NW) X(1, 16, NW) \
  X(2, 1, NW) X(2, 2, NW) X(2, 4, NW) X(2, 8, NW) X(2, 16, NW) \
  X(4, 1, NW) X(4, 2, NW) X(4, 4, NW) X(4, 8, NW) X(4, 16, NW) \
  X(8, 1, NW) X(8, 2, NW) X(8, 4, NW) X(8, 8, NW) \
  X(16, 1, NW) X(16, 2, NW) X(16, 4, NW)

static SparseFn pick_sparse(const Plan& p) {
#define SC_CASE(KK, OO, WW) if (p.K == KK && p.OCW == OO && p.NW == WW) return sparse_direct_fwd<KK, OO, WW>;
  SC_FOR_EACH_KO(SC_CASE, 8)
  SC_FOR_EACH_KO(SC_CASE, 16)
#undef SC_CASE
  return nullptr;
}

static hipError_t allow_lds(const void* fn, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int grid_size(const Plan& p, long long units, int* err) {
  *err = 0;
  const void* fn = reinterpret_cast<const void*>(pick_sparse(p));
  if (!fn) {
    *err = (int)hipErrorInvalidDeviceFunction;
    return 0;
  }
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = allow_lds(fn, p.lds_bytes);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, p.NW * 64, p.lds_bytes);
  if (e != hipSuccess) {
    *err = (int)e;
    return 0;
  }
  const long long slots = (long long)cus * (per_cu > 0 ? per_cu : 1);
  return (int)(units < slots ? units : slots);
}

int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks) {
  SparseFn fn = pick_sparse(p);
  if (!fn) return (int)hipErrorInvalidDeviceFunction;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), p.lds_bytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fn, dim3(nblocks), dim3(p.NW * 64), p.lds_bytes, reinterpret_cast<hipStream_t>(stream), a,
                     a.x, a.y, reinterpret_cast<const uint2*>(a.ent), a.seg, a.slot_row);
  return (int)hipGetLastError();
}

}  // namespace sc
