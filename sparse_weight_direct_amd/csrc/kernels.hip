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
//   staging  - each step's input (the exact range of every stride-phase plane the tile
//              reads, zero padding included) is copied HBM -> LDS by direct buffer loads
//              into LDS (gfx950 LDS DMA) into a ring of D slots, D-1 steps ahead of the
//              one being computed.  The (64-word block, channel) loads of a step are split
//              evenly over the wavefronts in block-major order; a block's per-lane source
//              offsets serve every channel (only a scalar offset of c*H*W words changes),
//              and padding words get an out-of-range offset, which the load turns into 0.
//              Every wavefront issues the same number of loads per step (padding with
//              repeats of an identical load), so a counted vmcnt wait finds its step;
//   compute  - each wavefront walks the non-zeros of its output-channel slots for the
//              step.  Its block of {enc, value} non-zeros is staged into the same ring slot
//              by the same loads; the wavefront reads it 64 entries at a time (one per
//              lane) and broadcasts each entry with v_readlane.  Per non-zero each lane
//              does one address add, K LDS reads 64 words apart and K fp32 FMAs;
//   store    - after a unit's last chunk, coalesced NCHW stores of the valid positions;
//              slots of channels without non-zeros store exact zeros.
// One barrier per step: before it, each wavefront waits (vmcnt) until its own loads of the
// step have landed; after it, the slot consumed in the previous step is refilled with the
// step D-1 ahead while this one is computed.
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

// The same with 16 bytes per lane (gfx950): lane i writes the 4 dwords at byte voff + soff
// to LDS byte address lds + 16*i; the source must be 16-byte aligned.
__device__ __forceinline__ void lds_dma_dwordx4(v4i rsrc, const float* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
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

// s_waitcnt vmcnt(N) for a wave-uniform N in [0, 63] (gfx9 encoding: vmcnt bits [3:0] and
// [15:14]; expcnt and lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void waitvm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
#define SC_VM4(b) case b: waitvm<b>(); break; case b + 1: waitvm<b + 1>(); break; \
                  case b + 2: waitvm<b + 2>(); break; case b + 3: waitvm<b + 3>(); break;
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    SC_VM4(0) SC_VM4(4) SC_VM4(8) SC_VM4(12) SC_VM4(16) SC_VM4(20) SC_VM4(24) SC_VM4(28)
    SC_VM4(32) SC_VM4(36) SC_VM4(40) SC_VM4(44) SC_VM4(48) SC_VM4(52) SC_VM4(56) SC_VM4(60)
    default: waitvm<0>(); break;
  }
}
#undef SC_VM4

// Wait until at most `later` of this wavefront's loads are outstanding (the loads of the
// steps issued after the one about to be computed), then barrier.  The empty asm keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void step_barrier(int later) {
  wait_vmcnt(later);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Source byte offset of the lane's word in block blk of the staged channel layout of the
// tile starting at extended index I0 (channel term excluded), relative to channel 0 of the
// tile's first image n0; out of range for padding, positions past the last image and the
// slack at the end of a channel.  (Wide layout with 16-byte loads: block_voff16 below.)
__device__ __forceinline__ uint32_t block_voff(const KArgs& a, int I0, int n0, int blk, int lane) {
  const int w = 64 * blk + lane;
  const int ph = w / a.PL;
  uint32_t off = kOutOfRange;
  if (ph < a.st * a.st) {
    const int J = I0 + (w - ph * a.PL);
    const int n = J / a.img_ext;
    const int rem = J - n * a.img_ext;
    const int t = rem / a.Pp;
    const int py = ph / a.st;
    const int y = t * a.st + py - a.pad;
    const int x = (rem - t * a.Pp) * a.st + (ph - py * a.st) - a.xoff;
    if (n < a.N && y >= 0 && y < a.H && x >= 0 && x < a.W)
      off = 4u * (uint32_t)(((n - n0) * a.C * a.H + y) * a.W + x);
  }
  return off;
}

// Wide layout (stride 1): source byte offset of the lane's 4 words in block sb of 256 words;
// the 4 words are one aligned group of 4 input words or 4 zeros.
__device__ __forceinline__ uint32_t block_voff16(const KArgs& a, int I0, int n0, int sb, int lane) {
  const int w = 256 * sb + 4 * lane;
  uint32_t off = kOutOfRange;
  if (w < a.PL) {
    const int J = I0 + w;
    const int n = J / a.img_ext;
    const int rem = J - n * a.img_ext;
    const int t = rem / a.Pp;
    const int y = t - a.pad;
    const int x = rem - t * a.Pp - a.xoff;
    if (n < a.N && y >= 0 && y < a.H && x >= 0 && x < a.W)
      off = 4u * (uint32_t)(((n - n0) * a.C * a.H + y) * a.W + x);
  }
  return off;
}

// Issue one step's loads into a ring slot: the wavefront's block of non-zeros (QE 16-byte
// loads of 128 entries, contiguous per wavefront), then its share [p0, p1) of the step's
// (block, channel) loads in block-major order (blocks of 256 words with 16-byte loads, or
// of 64 words), then repeats of its first non-zero load up to QB loads in all.  Channels
// at or past C (last chunk) are not loaded.
template <int T>
__device__ __forceinline__ void stage_step(const KArgs& a, const uint2* __restrict__ ent, int b0, int b1,
                                           v4i rsrc, int I0, int n0, int c0, int p0, int p1, float* slot,
                                           int wave, int lane) {
  const v4i ersrc = make_rsrc(ent + b0, (uint32_t)(b1 - b0) * 8u);
  float* edst = slot + a.nin + wave * (256 * a.QE);
  for (int q = 0; q < a.QE; q++) lds_dma_dwordx4(ersrc, edst + 256 * q, 16u * (64 * q + lane), 0u);
  const int ncl = __builtin_amdgcn_readfirstlane(min(a.Cc, a.C - c0));
  int issued = a.QE;
  const int bw = a.wide16 ? 256 : 64;
  int blk = p0 / a.Cc;
  int cl = p0 - blk * a.Cc;
  int p = p0;
  while (p < p1) {
    const uint32_t voff = a.wide16 ? block_voff16(a, I0, n0, blk, lane) : block_voff(a, I0, n0, blk, lane);
    const int cend = min(a.Cc, cl + (p1 - p));  // channels of this block in the share
    const int cstop = min(cend, ncl);
    const float* dst = slot + blk * bw + cl * a.CHS;
    uint32_t soff = 4u * (uint32_t)((c0 + cl) * a.HW);
    if (a.wide16) {
      for (int c = cl; c < cstop; c++) {
        lds_dma_dwordx4(rsrc, dst, voff, soff);
        dst += a.CHS;
        soff += 4u * (uint32_t)a.HW;
      }
    } else {
      for (int c = cl; c < cstop; c++) {
        lds_dma_dword(rsrc, dst, voff, soff);
        dst += a.CHS;
        soff += 4u * (uint32_t)a.HW;
      }
    }
    issued += cstop - cl;
    p += cend - cl;
    cl = 0;
    blk++;
  }
  if (a.D > 2)
    for (; issued < a.QB; issued++) lds_dma_dwordx4(ersrc, edst, 16u * lane, 0u);
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
      const int f = rem - e * a.Pp - a.cshift;
      if (e < a.E && f >= 0 && f < a.F) ob[b] = (n * a.M * a.E + e) * a.F + f;
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

// One step: the wavefront's slots and their non-zeros of this chunk, read from the block
// staged in the ring slot: header entries {count of slot o, 0} (OCW of them, rounded up to
// an even number), then the slots' non-zeros {enc, value} in slot order, each slot's run
// padded to an even length with zero-weight entries so that it is walked in pairs that
// never straddle a group of 64 (lane i holds entry i of the group).  The walk is split in
// slot ranges [O0, O1) so that the caller can issue staging loads between them; after(o)
// runs once slot o's run is done.
struct Walk {
  const uint32_t* eb;  // the wavefront's entries in the ring slot
  uint2 head;          // entries 0..63 (the header in lanes 0..OCW-1)
  uint2 cur;           // the current group of 64 entries
  int r;               // next entry's lane within the current group
  int base;            // entry index of the current group's lane 0
};

template <int NW>
__device__ __forceinline__ uint2 walk_group(const KArgs& a, const Walk& w, int base, int lane) {
  const int e = min(base + lane, 128 * a.QE - 1);
  return *reinterpret_cast<const uint2*>(w.eb + 2 * e);
}

template <int OCW, int NW>
__device__ __forceinline__ Walk walk_begin(const KArgs& a, const float* slot, int wave, int lane) {
  Walk w;
  w.eb = reinterpret_cast<const uint32_t*>(slot + a.nin) + wave * (256 * a.QE);
  w.head = walk_group<NW>(a, w, 0, lane);
  w.cur = w.head;
  w.r = (OCW + 1) & ~1;
  w.base = 0;
  return w;
}

template <int K, int OCW, int NW, int O0, int O1, typename After>
__device__ __forceinline__ void walk_slots(const KArgs& a, Walk& w, float (&acc)[OCW][K], const float* lane_lds,
                                           int lane, After&& after) {
#pragma unroll
  for (int o = O0; o < O1; o++) {
    int n = __builtin_amdgcn_readlane((int)w.head.x, o);  // even
    while (n > 0) {
      if (w.r == 64) {
        w.base += 64;
        w.cur = walk_group<NW>(a, w, w.base, lane);
        w.r = 0;
      }
      const int take = min(n, 64 - w.r);
      run_pairs<K>(acc[o], lane_lds, w.cur, w.r, take >> 1);
      w.r += take;
      n -= take;
    }
    after(o);
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
  int* bst = reinterpret_cast<int*>(lds + a.D * a.slot_words);

  const int b = xcd_logical(blockIdx.x, gridDim.x);
  const long long units = (long long)a.ntiles * a.G;
  const int u0 = (int)(units * b / gridDim.x);
  const int u1 = (int)(units * (b + 1) / gridDim.x);
  const int S = (u1 - u0) * a.nch;
  if (S == 0) return;

  for (int i = threadIdx.x; i < a.G * NW * (a.nch + 1); i += T) bst[i] = bstart[i];
  __syncthreads();

  // this wavefront's share of a step's (block, channel) loads
  const int P = a.nsb * a.Cc;
  const int p0 = __builtin_amdgcn_readfirstlane((int)((long long)P * wave / NW));
  const int p1 = __builtin_amdgcn_readfirstlane((int)((long long)P * (wave + 1) / NW));

  // issue side: the next step to stage (unit = tile * G + g, chunk is_k, ring slot is_buf)
  int is_tile = u0 / a.G, is_g = u0 - (u0 / a.G) * a.G, is_k = 0, is_buf = 0, is_new_tile = 1;
  int is_I0 = 0, is_n0 = 0;
  v4i rsrc = make_rsrc(x, 0u);
  auto issue = [&]() {
    if (is_new_tile) {
      is_I0 = is_tile * (64 * K);
      is_n0 = is_I0 / a.img_ext;
      const long long first = (long long)is_n0 * a.C * a.HW;
      rsrc = make_rsrc(x + first, (uint32_t)min((a.x_words - first) * 4, 0x7ffffff0LL));
      is_new_tile = 0;
    }
    const int* bw = bst + (is_g * NW + wave) * (a.nch + 1) + is_k;
    stage_step<T>(a, ent, bw[0], bw[1], rsrc, is_I0, is_n0, is_k * a.Cc, p0, p1, lds + is_buf * a.slot_words,
                  wave, lane);
    if (++is_buf == a.D) is_buf = 0;
    if (++is_k == a.nch) {
      is_k = 0;
      if (++is_g == a.G) {
        is_g = 0;
        is_tile++;
        is_new_tile = 1;
      }
    }
  };
  for (int s = 0; s < a.D - 1 && s < S; s++) issue();

  float acc[OCW][K];
#pragma unroll
  for (int o = 0; o < OCW; o++)
#pragma unroll
    for (int q = 0; q < K; q++) acc[o][q] = 0.0f;

  int tile = u0 / a.G, g = u0 - (u0 / a.G) * a.G, ck = 0, cbuf = 0;
  int drained = 0;  // a unit's stores were issued since the last wait: wait for everything
  for (int s = 0; s < S; s++) {
    // loads issued after step s's: those of steps s+1 .. min(s+D-2, S-1)
    const int later = drained ? 0 : a.QB * min(a.D - 2, S - 1 - s);
    step_barrier(later);  // step s landed; every wavefront is done with step s-1's slot
    drained = 0;
    const bool more = s + a.D - 1 < S;
    if (more && !a.issue_late) issue();
    const float* slot = lds + cbuf * a.slot_words;
    Walk w = walk_begin<OCW, NW>(a, slot, wave, lane);
    walk_slots<K, OCW, NW, 0, OCW>(a, w, acc, slot + lane, lane, [](int) {});
    // issued late, the loads of step s+D-1 overlap the wait at the next barrier; their
    // slot held step s-1, which every wavefront finished before this step's barrier
    if (more && a.issue_late) issue();
    if (ck + 1 == a.nch) {
      int ob[K];
      output_bases<K>(a, tile * (64 * K), lane, ob);
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
      drained = 1;
    }
    if (++cbuf == a.D) cbuf = 0;
    if (++ck == a.nch) {
      ck = 0;
      if (++g == a.G) {
        g = 0;
        tile++;
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
