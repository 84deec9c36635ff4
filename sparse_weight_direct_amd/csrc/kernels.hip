// gfx950 kernel: sparse direct convolution (the dense direct baseline is the same kernel
// on a handle that stores every filter tap).
//
// Work decomposition.  A tile is 64*K consecutive extended output positions (plan.h); a
// work unit is one tile for one group of output channels.  The grid is persistent: every
// CU runs the workgroups its LDS and registers allow, and each workgroup owns one
// contiguous run of units (runs differ by at most one unit), so neighbouring tiles, whose
// staged ranges overlap, are handled by the same workgroup one after the other.
//
// Per workgroup the units are walked as a stream of steps (unit, chunk of Cc input
// channels) through a ring of D LDS slots, by two roles that synchronise only through
// counters in LDS (no workgroup barrier inside the stream):
//   producer - one wavefront copies each step's input (the exact range of every
//              stride-phase plane the tile reads, zero padding included) HBM -> LDS with
//              direct buffer loads into LDS (gfx950 LDS DMA), into the slot of the step D
//              before it once every consumer has released that slot (done counter), and
//              publishes the step (ready counter) once its loads have landed.  A block's
//              per-lane source offsets serve every channel (only a scalar offset of c*H*W
//              words changes); padding words get an out-of-range offset, which the load
//              turns into 0;
//   consumers - the other wavefronts each own OCW output-channel slots.  A consumer waits
//              for the step's ready counter and walks its slots over its own block of
//              non-zeros for the step, which it loads from global memory 64 entries at a
//              time (one per lane, one group ahead of the walk) and broadcasts entry by
//              entry with v_readlane.  Per non-zero each lane does one address add, K LDS
//              reads 64 words apart and K fp32 FMAs.  (Quad plans walk differently: four
//              consecutive positions per lane and entries read from LDS, see the quad walk
//              below.)  It then releases the slot (done counter).  An entry is 8 bytes {LDS offset, fp32 weight}, or 4 bytes
//              {LDS offset, fp16 weight} for filter banks packed in the 32-bit word form
//              (the fp16 weight is widened to fp32 before the FMAs);
//   store    - after a unit's last chunk, each consumer stores its valid positions with
//              coalesced NCHW stores; slots of channels without non-zeros store exact zeros.
//              A row split over several consumers (pieces) is summed first: later pieces
//              leave partial sums in LDS buffers, the owner (piece 0) adds them in piece
//              order, so the result does not depend on timing.
// A consumer ahead of the others is held back only when it needs a step whose slot an
// earlier step still occupies, so per-step imbalance between wavefronts averages out over
// the ring.  Every wait on a counter is bounded (kSpinLimit sleeps), so a wavefront can
// never wait forever.
//
// Prior art kept from the pages: the input tile plus halo staged once per block and reused
// by every output channel, the packed per-non-zero word, and per-thread register
// accumulators (Tuteja et al., Sec. 5.1-5.5); the wave-uniform weight with lanes over
// consecutive output positions (the thread-per-output dataflow of "Escoin").
#include <hip/hip_runtime.h>

#include <type_traits>

#include "plan.h"
#include "xcd.h"

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

// Bounded wait until the LDS counter *p reaches target (every lane reads the same word).
// a.spin_limit sleeps of about 64 cycles (2^22 by default: far beyond any real wait).  A
// wait that gives up sets bit 0 of the handle's device status word (a vector global atomic
// from lane 0), so a synchronisation failure is reported (sparseconv_device_status) instead
// of passing as a plausible result; the wavefront then carries on, so every kernel ends.
__device__ __forceinline__ void lds_wait_ge(const uint32_t* p, uint32_t target, const KArgs& a) {
  int i = 0;
  for (; i < a.spin_limit; i++) {
    if (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (i == a.spin_limit && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// The same offsets for consecutive blocks blk, blk+1, ... without divisions: the lane's
// position (phase ph, word j of the phase plane, image n, row t, column x of the extended
// plane) advances by 64 words per block.  When PL is a multiple of 64 (stride > 1), a step
// into the next phase plane lands on word j = lane again, whose position is kept from
// init; otherwise that step, and images smaller than two blocks, fall back to the
// divisions.  (Producer only: narrow layout with more blocks than it caches.)
struct VoffIter {
  int w, ph, j, n, t, x;
  int n_s, t_s, x_s;  // position of word j = lane of a phase plane
  int q64, r64;       // 64 = q64 * Pp + r64
  __device__ __forceinline__ void full(const KArgs& a, int I0) {
    ph = w / a.PL;
    j = w - ph * a.PL;
    const int J = I0 + j;
    n = J / a.img_ext;
    const int rem = J - n * a.img_ext;
    t = rem / a.Pp;
    x = rem - t * a.Pp;
  }
  __device__ __forceinline__ void init(const KArgs& a, int I0, int blk, int lane) {
    w = 64 * blk + lane;
    q64 = 64 / a.Pp;
    r64 = 64 - q64 * a.Pp;
    const int J = I0 + lane;
    n_s = J / a.img_ext;
    const int rem = J - n_s * a.img_ext;
    t_s = rem / a.Pp;
    x_s = rem - t_s * a.Pp;
    full(a, I0);
  }
  __device__ __forceinline__ void next(const KArgs& a, int I0) {
    w += 64;
    j += 64;
    if (a.img_ext < 128) {
      full(a, I0);
      return;
    }
    if (j >= a.PL) {
      if ((a.PL & 63) == 0) {  // next phase plane, word j = lane
        ph++;
        j -= a.PL;
        n = n_s;
        t = t_s;
        x = x_s;
      } else {
        full(a, I0);
      }
      return;
    }
    x += r64;
    t += q64;
    if (x >= a.Pp) {
      x -= a.Pp;
      t++;
    }
    if (t >= a.HYp) {  // q64 + 1 < HYp here, so at most one image boundary is crossed
      t -= a.HYp;
      n++;
    }
  }
  __device__ __forceinline__ uint32_t off(const KArgs& a, int n0) const {
    if (ph >= a.st * a.st) return kOutOfRange;
    const int py = ph / a.st;
    const int y = t * a.st + py - a.pad;
    const int xx = x * a.st + (ph - py * a.st) - a.xoff;
    if (n < a.N && y >= 0 && y < a.H && xx >= 0 && xx < a.W)
      return 4u * (uint32_t)(((n - n0) * a.C * a.H + y) * a.W + xx);
    return kOutOfRange;
  }
};

// Floor division by a positive divisor for a numerator of either sign.
__device__ __forceinline__ int floor_div(int n, int d) { return n >= 0 ? n / d : -((d - 1 - n) / d); }

// Narrow layout with stride > 1 (PL a multiple of 64, images of at least 128 words): the
// lane's source offsets for every block of a channel in order, with additions and compares
// only (integer multiplies and divisions are quarter rate and the producer is a single
// wavefront).  Each phase plane (py, px) starts at word j = lane, whose image n, phase row t
// and phase column x are found once per tile; the source word of (n, t, x) in phase
// (py, px) is (n - n0)*C*H*W + (t*st + py - pad)*W + x*st + px - xoff, a linear function that
// is stepped with the position.  A word is in range when n < N and t, x fall inside the
// phase's rows and columns of the image.
struct PlaneIter {
  int n, t, x, src;      // current position and its source word offset
  int ns, ts, xs, srcs;  // position of word j = lane in phase (0, 0)
  int bi, py, px;        // block within the phase plane, phase
  int tlo, thi, xlo, xhi;
  __device__ __forceinline__ void bounds(const KArgs& a) {
    tlo = max(0, floor_div(a.pad - py + a.st - 1, a.st));
    thi = floor_div(a.H - 1 + a.pad - py, a.st);
    xlo = max(0, floor_div(a.xoff - px + a.st - 1, a.st));
    xhi = floor_div(a.W - 1 + a.xoff - px, a.st);
  }
  __device__ __forceinline__ void init(const KArgs& a, int I0, int n0, int lane) {
    const int J = I0 + lane;
    ns = J / a.img_ext;
    const int rem = J - ns * a.img_ext;
    ts = rem / a.Pp;
    xs = rem - ts * a.Pp;
    srcs = ((ns - n0) * a.C * a.H + ts * a.st - a.pad) * a.W + xs * a.st - a.xoff;
    bi = 0;
    py = 0;
    px = 0;
    n = ns;
    t = ts;
    x = xs;
    src = srcs;
    bounds(a);
  }
  __device__ __forceinline__ uint32_t off(const KArgs& a) const {
    const bool in = n < a.N && t >= tlo && t <= thi && x >= xlo && x <= xhi;
    return in ? 4u * (uint32_t)src : kOutOfRange;
  }
  // dT, dX: 64 = dT * Pp + dX; s1, s2, s3: source steps of 64 words, of a column wrap and of
  // an image wrap
  __device__ __forceinline__ void next(const KArgs& a, int nbp, int dT, int dX, int s1, int s2, int s3) {
    if (++bi == nbp) {  // next phase plane
      bi = 0;
      if (++px == a.st) {
        px = 0;
        py++;
      }
      n = ns;
      t = ts;
      x = xs;
      src = srcs + py * a.W + px;
      bounds(a);
      return;
    }
    x += dX;
    t += dT;
    src += s1;
    if (x >= a.Pp) {
      x -= a.Pp;
      t++;
      src += s2;
    }
    if (t >= a.HYp) {  // at most one image boundary per block (images of >= 128 words)
      t -= a.HYp;
      n++;
      src += s3;
    }
  }
};

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

// Producer: issue the input loads of one step (channels [c0, c0 + ncl) of a tile) into a
// ring slot, block by block (blocks of 256 words with 16-byte loads, or of 64 words), and
// call first_done(ncl) once the first block's ncl loads are issued.  Returns the number of
// loads issued.  voff0..voff3 hold the first blocks' offsets for the tile; further blocks
// are computed on the fly.
template <typename FirstDone>
__device__ __forceinline__ int stage_rows(const KArgs& a, v4i rsrc, int I0, int n0, int c0, int ncl,
                                          const uint32_t (&voffc)[4], float* slot, int lane,
                                          FirstDone&& first_done) {
  const int bw = a.wide16 ? 256 : 64;
  // narrow layout, stride > 1: additions-only stepping through the phase planes
  const bool planes = !a.wide16 && a.st > 1 && (a.PL & 63) == 0 && a.img_ext >= 128;
  const int nbp = a.PL >> 6;
  const int dT = 64 / a.Pp, dX = 64 - dT * a.Pp;
  const int s1 = dT * a.st * a.W + dX * a.st;
  const int s2 = a.st * a.W - a.Pp * a.st;
  const int s3 = a.C * a.H * a.W - a.HYp * a.st * a.W;
  PlaneIter pi;
  if (planes) pi.init(a, I0, n0, lane);
  VoffIter vi;
  if (!planes && !a.wide16 && a.nsb > 4) vi.init(a, I0, 4, lane);
  for (int blk = 0; blk < a.nsb; blk++) {
    // explicit selects keep the cached offsets in registers (no indexed private array)
    uint32_t voff;
    if (planes) {
      if (blk > 0) pi.next(a, nbp, dT, dX, s1, s2, s3);
      voff = pi.off(a);
    } else if (blk < 4) {
      voff = blk == 0 ? voffc[0] : blk == 1 ? voffc[1] : blk == 2 ? voffc[2] : voffc[3];
    } else if (a.wide16) {
      voff = block_voff16(a, I0, n0, blk, lane);
    } else {
      if (blk > 4) vi.next(a, I0);
      voff = vi.off(a, n0);
    }
    const float* dst = slot + blk * bw;
    uint32_t soff = 4u * (uint32_t)(c0 * a.HW);
    if (a.wide16) {
      for (int c = 0; c < ncl; c++) {
        lds_dma_dwordx4(rsrc, dst, voff, soff);
        dst += a.CHS;
        soff += 4u * (uint32_t)a.HW;
      }
    } else {
      for (int c = 0; c < ncl; c++) {
        lds_dma_dword(rsrc, dst, voff, soff);
        dst += a.CHS;
        soff += 4u * (uint32_t)a.HW;
      }
    }
    if (blk == 0) first_done(ncl);
  }
  return a.nsb * ncl;
}

// Output word offset (without the channel term) of each of the lane's K store positions, or
// -1.  Store b of the lane writes position I0 + lane + 64 b, or in a quad plan
// I0 + 252 (b / 4) + lane + 64 (b % 4) (positions past 251 of a block are lane 63's junk):
// quad results are transposed through LDS first, so that the stores stay lane-consecutive.
template <int K, bool Q>
__device__ __forceinline__ void output_bases(const KArgs& a, int I0, int lane, int (&ob)[K]) {
#pragma unroll
  for (int b = 0; b < K; b++) {
    const int in_block = lane + 64 * (Q ? (b & 3) : b);
    const long long I = Q ? (long long)I0 + kQuadBlock * (b >> 2) + in_block : (long long)I0 + in_block;
    ob[b] = -1;
    if ((!Q || in_block < kQuadBlock) && I < a.ext_total) {
      const int Ii = (int)I;
      const int n = Ii / a.img_ext;
      const int rem = Ii - n * a.img_ext;
      const int e = rem / a.Pp;
      const int f = rem - e * a.Pp - a.cshift;
      if (e < a.E && f >= 0 && f < a.F) ob[b] = (n * a.M * a.E + e) * a.F + f;
    }
  }
}

// Entry formats of the kernel stream.  A group of 64 entries is held one per lane; header
// entries hold a slot's count in their first (or only) word.
struct EntF32 {  // 8 bytes: {LDS word offset, fp32 weight bits}
  using T = uint2;
  static __device__ __forceinline__ T zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ int count(T g, int o) { return __builtin_amdgcn_readlane((int)g.x, o); }
  static __device__ __forceinline__ void get(T g, int l, uint32_t& off, float& w) {
    off = (uint32_t)__builtin_amdgcn_readlane((int)g.x, l);
    w = __int_as_float(__builtin_amdgcn_readlane((int)g.y, l));
  }
};
// 4 bytes: fp16 weight bits in bits 15..0, LDS word offset in bits 31..16 (one v_readlane
// per entry; the conversion reads the low half directly)
struct EntH16 {
  using T = uint32_t;
  static __device__ __forceinline__ T zero() { return 0u; }
  static __device__ __forceinline__ int count(T g, int o) { return __builtin_amdgcn_readlane((int)g, o); }
  static __device__ __forceinline__ void get(T g, int l, uint32_t& off, float& w) {
    const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)g, l);
    off = e >> 16;
    w = (float)__builtin_bit_cast(_Float16, (unsigned short)(e & 0xffffu));
  }
};

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
template <int K, typename EF>
__device__ __forceinline__ void pair(float (&acc)[K], const float* lane_lds, const typename EF::T grp, int l) {
  uint32_t o0, o1;
  float w0, w1;
  EF::get(grp, l, o0, w0);
  EF::get(grp, l + 1, o1, w1);
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

// n consecutive non-zeros starting at lane l of a group: pairs, then a single one if n is odd.
template <int K, typename EF>
__device__ __forceinline__ void run_entries(float (&acc)[K], const float* lane_lds, const typename EF::T grp, int l,
                                            int n) {
  const int lend = l + (n & ~1);
  if (n & 2) {
    pair<K, EF>(acc, lane_lds, grp, l);
    l += 2;
  }
  for (; l < lend; l += 4) {
    pair<K, EF>(acc, lane_lds, grp, l);
    pair<K, EF>(acc, lane_lds, grp, l + 2);
  }
  if (n & 1) {
    uint32_t o;
    float w;
    EF::get(grp, lend, o, w);
    fma_entry<K>(acc, lane_lds, o, w);
  }
}

// One step: the wavefront's slots and their non-zeros of this chunk, from its block of the
// stream: header entries holding the count of slot o (OCW of them, rounded up to an even
// number), then the slots' non-zeros in slot order, walked in pairs (and a single last
// one for an odd run) that never straddle a group of 64 (lane i holds entry i of the
// group).  Blocks start at multiples of 64 entries, so a block is a whole number of groups;
// the groups arrive in registers from the caller (next_group), which loads them one group
// ahead straight from the stream in global memory.
template <typename EF>
struct Walk {
  typename EF::T head;  // the block's first group (the header in lanes 0..OCW-1)
  typename EF::T cur;   // the current group of 64 entries
  int r;                // next entry's lane within the current group
};

template <int K, int OCW, typename EF, typename NextGroup>
__device__ __forceinline__ void walk_slots(Walk<EF>& w, float (&acc)[OCW][K], const float* lane_lds,
                                           NextGroup&& next_group) {
#pragma unroll
  for (int o = 0; o < OCW; o++) {
    int n = EF::count(w.head, o);
    while (n > 0) {
      if (w.r == 64) {
        w.cur = next_group();
        w.r = 0;
      }
      const int take = min(n, 64 - w.r);
      run_entries<K, EF>(acc[o], lane_lds, w.cur, w.r, take);
      w.r += take;
      n -= take;
    }
  }
}

// Quad walk (quad plans).  Lane l holds positions 4l..4l+3 of two blocks 252 words apart.
// A non-zero whose LDS offset is enc reads, per block, the aligned quad at word
// 4l + (enc & ~3) (one 16-byte read) and needs its words j + cls (cls = enc & 3) for
// positions j: words past 3 are words j + cls - 4 of the next lane's quad, which a DPP FMA
// (wave_shl:1) takes from lane l + 1.  A slot's non-zeros of a chunk come sorted by class,
// so each class is a run with a fixed FMA pattern.  Entries {byte offset of the aligned
// quad, fp32 weight} are read by the whole wave from the consumer's entry ring in LDS (one
// broadcast read, no v_readlane), and the walk is pipelined: the quads of the next
// non-zero and the entry after it are read before the current non-zero's FMAs.
typedef float v4f __attribute__((ext_vector_type(4)));

// the DPP FMAs of one non-zero of class C (C = 1..3): acc[4b + 4 - C + i] += w * word i of
// the next lane's quad b.  The s_nop gives the two wait states a DPP read needs after a
// vector write of any of its registers.
template <int C>
__device__ __forceinline__ void quad_dpp(float (&A)[8], const v4f q0, const v4f q1, float w) {
  if constexpr (C == 1) {
    asm volatile("s_nop 1\n"
                 "v_fmac_f32_dpp %0, %2, %4 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %1, %3, %4 wave_shl:1 row_mask:0xf bank_mask:0xf"
                 : "+v"(A[3]), "+v"(A[7])
                 : "v"(q0.x), "v"(q1.x), "v"(w));
  } else if constexpr (C == 2) {
    asm volatile("s_nop 1\n"
                 "v_fmac_f32_dpp %0, %4, %8 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %1, %5, %8 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %2, %6, %8 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %3, %7, %8 wave_shl:1 row_mask:0xf bank_mask:0xf"
                 : "+v"(A[2]), "+v"(A[3]), "+v"(A[6]), "+v"(A[7])
                 : "v"(q0.x), "v"(q0.y), "v"(q1.x), "v"(q1.y), "v"(w));
  } else if constexpr (C == 3) {
    asm volatile("s_nop 1\n"
                 "v_fmac_f32_dpp %0, %6, %12 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %1, %7, %12 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %2, %8, %12 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %3, %9, %12 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %4, %10, %12 wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 "v_fmac_f32_dpp %5, %11, %12 wave_shl:1 row_mask:0xf bank_mask:0xf"
                 : "+v"(A[1]), "+v"(A[2]), "+v"(A[3]), "+v"(A[5]), "+v"(A[6]), "+v"(A[7])
                 : "v"(q0.x), "v"(q0.y), "v"(q0.z), "v"(q1.x), "v"(q1.y), "v"(q1.z), "v"(w));
  }
}

// The 8 FMAs of one non-zero of class C.
template <int C>
__device__ __forceinline__ void quad_fma(float (&A)[8], const v4f q0, const v4f q1, float w) {
#pragma unroll
  for (int j = 0; j + C < 4; j++) {
    A[j] = fmaf(w, q0[j + C], A[j]);
    A[4 + j] = fmaf(w, q1[j + C], A[4 + j]);
  }
  quad_dpp<C>(A, q0, q1, w);
}

// Pipeline state between runs: the quads and weight of the current non-zero (reads in
// flight), the entry after it (read in flight) and the index of the entry after that.
struct QuadPipe {
  v4f q0, q1;
  float w;
  uint2 en;
  int i;
};

// lb: the lane's byte address of its first quad in the slot (slot + 16 lane).
__device__ __forceinline__ void quad_read(const char* lb, uint32_t off, v4f& q0, v4f& q1) {
  q0 = *reinterpret_cast<const v4f*>(lb + off);
  q1 = *reinterpret_cast<const v4f*>(lb + off + 4 * kQuadBlock);
}

// A run of n non-zeros of class C into the slot's accumulators A.  fetch(i) returns entry i
// of the step's block (already in the ring); the two zero entries that close every block
// keep the one-ahead reads of the block's last run inside the block.
template <int C, typename Fetch>
__device__ __forceinline__ void quad_run(float (&A)[8], QuadPipe& p, const char* lb, int n, Fetch&& fetch) {
  for (; n >= 2; n -= 2) {
    v4f b0, b1;
    quad_read(lb, p.en.x, b0, b1);
    const float wb = __uint_as_float(p.en.y);
    p.en = fetch(p.i++);
    quad_fma<C>(A, p.q0, p.q1, p.w);
    quad_read(lb, p.en.x, p.q0, p.q1);
    p.w = __uint_as_float(p.en.y);
    p.en = fetch(p.i++);
    quad_fma<C>(A, b0, b1, wb);
  }
  if (n) {
    quad_fma<C>(A, p.q0, p.q1, p.w);
    quad_read(lb, p.en.x, p.q0, p.q1);
    p.w = __uint_as_float(p.en.y);
    p.en = fetch(p.i++);
  }
}

// Step iterator over a workgroup's run of units: unit = tile * G + g, then chunk k.
struct StepIt {
  int tile, g, k;
  __device__ __forceinline__ void next(const KArgs& a) {
    if (++k == a.nch) {
      k = 0;
      if (++g == a.G) {
        g = 0;
        tile++;
      }
    }
  }
};

template <int K, int NW>
__device__ __forceinline__ void producer(const KArgs& a, const float* __restrict__ x, StepIt it, int S,
                                         uint32_t* ready, uint32_t* done, float* lds, int lane) {
  constexpr int NC = NW - 1;
  int cur_tile = -1, I0 = 0, n0 = 0;
  v4i rsrc = make_rsrc(x, 0u);
  uint32_t voffc[4] = {kOutOfRange, kOutOfRange, kOutOfRange, kOutOfRange};
  int pending = -1;  // the step whose loads were issued but not yet published
  for (int t = 0; t < S; t++) {
    const int buf = t % a.D;
    // the slot held step t - D: wait until every consumer has released it.  If that wait
    // would block, publish the pending step as soon as it has landed instead of after the
    // next issue, so that consumers ahead of the slowest one can start on it.
    if (t >= a.D) {
      const uint32_t target = (uint32_t)(NC * (t / a.D));
      if (pending >= 0 && __hip_atomic_load(&done[buf], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        wait_vmcnt(0);
        __hip_atomic_store(&ready[pending % a.D], (uint32_t)(pending / a.D + 1), __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
        pending = -1;
      }
      lds_wait_ge(&done[buf], target, a);
    }
    if (it.tile != cur_tile) {
      cur_tile = it.tile;
      I0 = cur_tile * a.tp;
      n0 = I0 / a.img_ext;
      const long long first = (long long)n0 * a.C * a.HW;
      rsrc = make_rsrc(x + first, (uint32_t)min((a.x_words - first) * 4, 0x7ffffff0LL));
#pragma unroll
      for (int i = 0; i < 4; i++)
        voffc[i] = a.wide16 ? block_voff16(a, I0, n0, i, lane) : block_voff(a, I0, n0, i, lane);
    }
    const int c0 = it.k * a.Cc;
    const int ncl = __builtin_amdgcn_readfirstlane(min(a.Cc, a.C - c0));
    // the previous step is published as soon as it has landed, which is once at most the
    // first block of this step is outstanding (the loads complete in order): the copy engine
    // keeps working on this step meanwhile
    stage_rows(a, rsrc, I0, n0, c0, ncl, voffc, lds + buf * a.slot_words, lane, [&](int issued) {
      if (pending >= 0) {
        wait_vmcnt(issued <= 63 ? issued : 0);
        __hip_atomic_store(&ready[pending % a.D], (uint32_t)(pending / a.D + 1), __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    });
    pending = t;
    it.next(a);
  }
  if (pending >= 0) {
    wait_vmcnt(0);
    __hip_atomic_store(&ready[pending % a.D], (uint32_t)(pending / a.D + 1), __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

template <int K, int OCW, int NW, typename EF, bool Q>
__device__ __forceinline__ void consumer(const KArgs& a, float* __restrict__ y, const typename EF::T* __restrict__ ent,
                                         const int* bst, const int* __restrict__ slot_row,
                                         const int* __restrict__ slot_comb, StepIt it, int S, const uint32_t* ready,
                                         uint32_t* done, uint32_t* pfull, uint32_t* pcons, float* pbuf, float* lds,
                                         int c, int lane) {
  constexpr int NC = NW - 1;
  // The consumer's groups of 64 entries, in walk order (every group of a step's block, then
  // the next step's): cur is walked while nxt, the following group, is in flight.  Only one
  // load is outstanding at a time, apart from the output stores after a unit.
  StepIt pf = it;  // step of the group in nxt
  int pg = 0;      // its index within that step's block
  int pstep = 0;   // its step number in this workgroup's stream
  auto block = [&](const StepIt& p) -> const int* { return bst + (p.g * NC + c) * (a.nch + 1) + p.k; };
  using ET = typename EF::T;
  auto load_group = [&]() -> ET { return pstep < S ? ent[block(pf)[0] + 64 * pg + lane] : EF::zero(); };
  auto advance = [&]() {
    const int* bw = block(pf);
    if (64 * (pg + 1) < bw[1] - bw[0]) {
      pg++;
    } else {
      pg = 0;
      pf.next(a);
      pstep++;
    }
  };
  ET nxt = load_group();  // group 0 of step 0
  auto next_group = [&]() -> ET {
    wait_vmcnt(0);
    const ET g = nxt;
    advance();
    nxt = load_group();
    return g;
  };
  ET first = next_group();  // step 0's first group; nxt holds the one after it
  float acc[OCW][K];
#pragma unroll
  for (int o = 0; o < OCW; o++)
#pragma unroll
    for (int q = 0; q < K; q++) acc[o][q] = 0.0f;
  int units_done = 0;  // units finished by this workgroup
  for (int s = 0; s < S; s++) {
    const int buf = s % a.D;
    lds_wait_ge(&ready[buf], (uint32_t)(s / a.D + 1), a);
    const float* slot = lds + buf * a.slot_words;
    if constexpr (Q) {
      // the consumer's entry ring: entry i of the step's block sits at i & 127.  Before
      // each run of at most 64 entries, the groups it reads are copied in (the ring half a
      // group overwrites held group g - 2, all of whose entries were read before the run),
      // so the run itself only reads LDS.
      uint2* ring = reinterpret_cast<uint2*>(lds + a.ring_words) + (threadIdx.x >> 6) * 128;
      ring[lane] = first;
      int gi = 0;
      auto ensure = [&](int last) {
        while (gi < (last >> 6)) {
          gi++;
          ring[((gi & 1) << 6) + lane] = next_group();
        }
      };
      auto fetch = [&](int i) -> uint2 { return ring[i & 127]; };
      const char* lb = reinterpret_cast<const char*>(slot) + 16 * lane;
      constexpr int H = (OCW + 1) & ~1;  // header entries: per slot, the four class counts
      QuadPipe qp;
      ensure(H + 1);
      const uint2 e0 = fetch(H);
      quad_read(lb, e0.x, qp.q0, qp.q1);
      qp.w = __uint_as_float(e0.y);
      qp.en = fetch(H + 1);
      qp.i = H + 2;
      auto run = [&](auto cls, float (&A)[8], int n) {
        while (n > 0) {
          const int t = min(n, 64);
          ensure(qp.i + t - 1);
          quad_run<decltype(cls)::value>(A, qp, lb, t, fetch);
          n -= t;
        }
      };
#pragma unroll
      for (int o = 0; o < OCW; o++) {
        const uint32_t c01 = (uint32_t)__builtin_amdgcn_readlane((int)first.x, o);
        const uint32_t c23 = (uint32_t)__builtin_amdgcn_readlane((int)first.y, o);
        run(std::integral_constant<int, 0>{}, acc[o], (int)(c01 & 0xffffu));
        run(std::integral_constant<int, 1>{}, acc[o], (int)(c01 >> 16));
        run(std::integral_constant<int, 2>{}, acc[o], (int)(c23 & 0xffffu));
        run(std::integral_constant<int, 3>{}, acc[o], (int)(c23 >> 16));
      }
    } else {
      Walk<EF> w;
      w.head = first;
      w.cur = first;
      w.r = (OCW + 1) & ~1;
      walk_slots<K, OCW, EF>(w, acc, slot + lane, next_group);
    }
    // every group of this step's block has been walked: nxt is the next step's first group
    if (s + 1 < S) first = next_group();
    // release the slot's input part (the walk's LDS reads are complete before the add);
    // one lane adds, so the counter advances by one per consumer
    uint32_t before = 0;
    if (lane == 0) before = __hip_atomic_fetch_add(&done[buf], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    // wave priority from this consumer's finishing rank on the step: the issue arbiter
    // favours older waves, so without this the highest-index consumers lag behind and
    // hold up the refill of their slots
    const int rank = __builtin_amdgcn_readfirstlane((int)(before - (uint32_t)(NC * (s / a.D))));
    if (rank >= NC - 4)
      __builtin_amdgcn_s_setprio(2);
    else if (2 * rank >= NC)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    if (it.k + 1 == a.nch) {
      // generation of this group's partial buffers: the group's units this workgroup has
      // finished (units cycle through the G groups, so every G-th unit is this group's)
      const int gen = units_done / a.G;
      const int* rows = slot_row + (it.g * NC + c) * OCW;
      const int* comb = slot_comb + (it.g * NC + c) * OCW;
      // later pieces of split rows leave their partial sums in LDS buffers (after the
      // previous unit's owner has read the buffer) ...
#pragma unroll
      for (int o = 0; o < OCW; o++) {
        const int v = rows[o];
        if (v <= -2) {
          const int b = -2 - v;
          lds_wait_ge(&pcons[b], (uint32_t)gen, a);
          float* pb = pbuf + b * (64 * K) + lane;
#pragma unroll
          for (int q = 0; q < K; q++) pb[64 * q] = acc[o][q];
          if (lane == 0)
            __hip_atomic_store(&pfull[b], (uint32_t)(gen + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
          for (int q = 0; q < K; q++) acc[o][q] = 0.0f;
        }
      }
      // ... and the owner of each row adds them in piece order, then stores
      int ob[K];
      output_bases<K, Q>(a, it.tile * a.tp, lane, ob);
      const int plane = a.E * a.F;
#pragma unroll
      for (int o = 0; o < OCW; o++) {
        const int row = rows[o];
        if (row >= 0) {
          const int cm = comb[o];
          for (int i = 0; i < (cm & 255); i++) {
            const int b = (cm >> 8) + i;
            lds_wait_ge(&pfull[b], (uint32_t)(gen + 1), a);
            const float* pb = pbuf + b * (64 * K) + lane;
#pragma unroll
            for (int q = 0; q < K; q++) acc[o][q] += pb[64 * q];
            if (lane == 0)
              __hip_atomic_store(&pcons[b], (uint32_t)(gen + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          // ordinary (write-back) stores: the partial 64-byte segments at output-row and tile
          // boundaries are merged in L2 instead of being written to HBM separately
          if constexpr (Q) {
            // a quad lane holds positions 4l..4l+3 of each block: transpose each block through
            // this consumer's entry ring (1 KB, idle once the unit's last walk is issued; the
            // wave's LDS accesses complete in order), then store position l + 64k from lane l
            float* tb = reinterpret_cast<float*>(lds + a.ring_words) + (threadIdx.x >> 6) * 256;
#pragma unroll
            for (int b = 0; b < 2; b++) {
              v4f v;
              v.x = acc[o][4 * b];
              v.y = acc[o][4 * b + 1];
              v.z = acc[o][4 * b + 2];
              v.w = acc[o][4 * b + 3];
              *reinterpret_cast<v4f*>(tb + 4 * lane) = v;
              float t[4];
#pragma unroll
              for (int k = 0; k < 4; k++) t[k] = tb[lane + 64 * k];
#pragma unroll
              for (int k = 0; k < 4; k++)
                if (ob[4 * b + k] >= 0) y[ob[4 * b + k] + row * plane] = t[k];
            }
          } else {
#pragma unroll
            for (int q = 0; q < K; q++)
              if (ob[q] >= 0) y[ob[q] + row * plane] = acc[o][q];
          }
        }
#pragma unroll
        for (int q = 0; q < K; q++) acc[o][q] = 0.0f;
      }
      units_done++;
    }
    it.next(a);
  }
}

// Pointers are separate restrict-qualified arguments so the compiler knows the streams
// are read-only.
template <int K, int OCW, int NW, typename EF, bool Q>
__global__ __launch_bounds__(NW * 64, 4) void sparse_direct_fwd(
    const KArgs a, const float* __restrict__ x, float* __restrict__ y,
    const typename EF::T* __restrict__ ent, const int* __restrict__ bstart,
    const int* __restrict__ slot_row, const int* __restrict__ slot_comb) {
  constexpr int T = NW * 64;
  constexpr int NC = NW - 1;
  extern __shared__ float lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* ready = reinterpret_cast<uint32_t*>(lds + a.D * a.slot_words);
  uint32_t* done = ready + kMaxDepth;
  int* bst = reinterpret_cast<int*>(done + kMaxDepth);
  uint32_t* pfull = reinterpret_cast<uint32_t*>(bst + a.G * NC * (a.nch + 1));  // split rows
  uint32_t* pcons = pfull + a.nbuf;
  float* pbuf = reinterpret_cast<float*>(pcons + a.nbuf);

  // adjacent runs of tiles, which share halo rows, on one XCD's L2
  const int b = xcd_logical(blockIdx.x, gridDim.x);
  const long long units = (long long)a.ntiles * a.G;
  const int u0 = (int)(units * b / gridDim.x);
  const int u1 = (int)(units * (b + 1) / gridDim.x);
  const int S = (u1 - u0) * a.nch;
  if (S == 0) return;

  if (threadIdx.x < 2 * kMaxDepth) ready[threadIdx.x] = 0u;
  for (int i = threadIdx.x; i < 2 * a.nbuf; i += T) pfull[i] = 0u;
  for (int i = threadIdx.x; i < a.G * NC * (a.nch + 1); i += T) bst[i] = bstart[i];
  __syncthreads();

  StepIt it{u0 / a.G, u0 - (u0 / a.G) * a.G, 0};
  if (wave == NC) __builtin_amdgcn_s_setprio(3);  // the producer must never starve
  if (wave == NC)
    producer<K, NW>(a, x, it, S, ready, done, lds, lane);
  else
    consumer<K, OCW, NW, EF, Q>(a, y, ent, bst, slot_row, slot_comb, it, S, ready, done, pfull, pcons, pbuf, lds,
                                wave, lane);
}

template <typename EF>
using SparseFn = void (*)(KArgs, const float*, float*, const typename EF::T*, const int*, const int*, const int*);

#define SC_FOR_EACH_KO(X, NW) \
  X(1, 1, NW) X(2, 1, NW) X(4, 1, NW) X(6, 1, NW) X(7, 1, NW) X(8, 1, NW) X(12, 1, NW) X(16, 1, NW) \
  X(1, 2, NW) X(2, 2, NW) X(4, 2, NW) X(6, 2, NW) X(7, 2, NW) X(8, 2, NW) X(12, 2, NW) X(16, 2, NW) \
  X(1, 3, NW) X(2, 3, NW) X(4, 3, NW) X(6, 3, NW) X(7, 3, NW) X(8, 3, NW) X(12, 3, NW) X(16, 3, NW) \
  X(1, 5, NW) X(2, 5, NW) X(4, 5, NW) X(6, 5, NW) X(7, 5, NW) X(8, 5, NW) X(12, 5, NW) \
  X(1, 9, NW) X(2, 9, NW) X(4, 9, NW) X(6, 9, NW) X(7, 9, NW)

template <typename EF>
static SparseFn<EF> pick_sparse(const Plan& p) {
  if (p.quad) {  // quad kernels: 8-byte entries, K = 8, 3/5/9 slots
    if constexpr (std::is_same<EF, EntF32>::value) {
      if (p.K == 8 && p.NW == 16) {
        if (p.OCW == 3) return sparse_direct_fwd<8, 3, 16, EF, true>;
        if (p.OCW == 5) return sparse_direct_fwd<8, 5, 16, EF, true>;
        if (p.OCW == 9) return sparse_direct_fwd<8, 9, 16, EF, true>;
      }
    }
    return nullptr;
  }
#define SC_CASE(KK, OO, WW) if (p.K == KK && p.OCW == OO && p.NW == WW) return sparse_direct_fwd<KK, OO, WW, EF, false>;
  SC_FOR_EACH_KO(SC_CASE, 16)
#undef SC_CASE
  return nullptr;
}

static const void* kernel_of(const Plan& p) {
  return p.h16 ? reinterpret_cast<const void*>(pick_sparse<EntH16>(p))
               : reinterpret_cast<const void*>(pick_sparse<EntF32>(p));
}

static hipError_t allow_lds(const void* fn, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int occupancy(const Plan& p, int* cus, int* per_cu) {
  *cus = 0;
  *per_cu = 0;
  const void* fn = kernel_of(p);
  if (!fn) return (int)hipErrorInvalidDeviceFunction;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = allow_lds(fn, p.lds_bytes);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, fn, p.NW * 64, p.lds_bytes);
  if (*per_cu < 1) *per_cu = 1;
  return (int)e;
}

template <typename EF>
static int launch_as(const Plan& p, const KArgs& a, void* stream, int nblocks) {
  SparseFn<EF> fn = pick_sparse<EF>(p);
  if (!fn) return (int)hipErrorInvalidDeviceFunction;
  hipError_t e = allow_lds(reinterpret_cast<const void*>(fn), p.lds_bytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fn, dim3(nblocks), dim3(p.NW * 64), p.lds_bytes, reinterpret_cast<hipStream_t>(stream), a,
                     a.x, a.y, reinterpret_cast<const typename EF::T*>(a.ent), a.seg, a.slot_row, a.slot_comb);
  return (int)hipGetLastError();
}

int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks) {
  return p.h16 ? launch_as<EntH16>(p, a, stream, nblocks) : launch_as<EntF32>(p, a, stream, nblocks);
}

}  // namespace sc
