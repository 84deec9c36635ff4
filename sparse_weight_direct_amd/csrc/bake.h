// Weights-in-code mapping ("baked" kernels): at pack time the filter bank of one layer is
// written into the instruction stream of a gfx950 kernel, every stored non-zero becoming
// one v_fmac_f32 whose multiplier is a 32-bit literal, with the output channel's
// accumulator and the filter tap's input register fixed in the instruction.  The kernel is
// assembled in-process (amd_comgr) and loaded as a code object (hipModuleLoadData).
//
// Why: unstructured sparsity gives every non-zero its own output channel and filter tap.
// A kernel that reads the weights as data must select both per non-zero at run time,
// which costs instructions, LDS reads or register-index changes for every FMA.  Fixed in
// the code, the selection costs nothing: per non-zero the wavefront issues exactly one
// VALU instruction, which does 64 FMAs (one per output position of its lanes).
//
// Work decomposition.  Output positions are numbered in an extended space of N*E*Pb
// positions, Pb = F + (S-1)/st: position q = (n*E + e)*Pb + f, junk where f >= F.  A
// wavefront takes V = 64 - (S-1)/st consecutive positions (lanes V..63 are junk) and one
// group of output channels, whose accumulators it keeps in VGPRs for the whole input.  It
// walks the input channel by channel and filter row by filter row (a "step" (c, r)); per
// step it loads, for each stride phase sp of the filter columns, the vector
// X[n, c, e*st - pad + r, f*st + sp - pad] over its lanes (zero where that lies in the
// padding: the offset is then out of the buffer's range), and obtains the taps s = sp +
// st*sq of the same row by shifting that vector sq lanes down (DPP wave_shl:1, repeated).
// Loads run a fixed number of steps ahead of the FMAs.  At the end every lane stores its
// valid positions of every output channel of the group (coalesced NCHW rows).
//
// The code is straight-line apart from the selection of the group's section at the start:
// there is no loop, so no wave can run away; the only memory accesses are the kernel
// argument load and buffer loads/stores whose descriptors bound them to the caller's input
// and output, so no address computed inside the kernel can reach other memory.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "plan.h"

namespace sc {

struct BakePlan {
  int G = 1;        // output-channel groups
  int Q = 1;        // channel splits: the input channels of a unit are split over Q wavefronts
                    // of one workgroup, whose partial sums are added through LDS
  int T = 4;        // units per workgroup (a workgroup is Q*T wavefronts)
  int D = 4;        // steps whose loads are in flight ahead of the FMAs
  int dpp = 1;      // 1: shifted taps by lane shifts; 0: one load per tap (V = 64)
  int perm = 1;     // lane shifts by ds_bpermute_b32 through the LDS crossbar (1) or by DPP
                    // moves on the VALU (0)
  int Pb = 0;       // extended row pitch F + maxsq
  int V = 64;       // valid positions per wavefront = 64 - maxsq
  int maxsq = 0;    // largest lane shift (S-1)/st (0 without DPP)
  int Mg = 0;       // accumulators per wavefront (largest group, padded to 4 when Q > 1)
  int vgprs = 0, sgprs = 0;
  int lds_bytes = 0;         // LDS per workgroup: partial sums of the channel splits, or the
                             // staged chunk buffers
  int rc = 0;                // channels per round of the split reduction (LDS per split: rc/4 KB)
  // staged plans (stride 1): a workgroup's T tiles of 64 lanes cover T*64 consecutive positions
  // of the padded layout (V = 64, pitch Pb = the layout's row pitch); per chunk of Cc channels
  // each channel's window (chs words) is copied into LDS once by LDS DMA (bw words per
  // instruction) into one of nbuf chunk buffers, nbuf - 1 chunks ahead of the FMAs, and every
  // tap is read from LDS at an immediate offset
  int stage = 0;
  int Cc = 0, chs = 0, bw = 0, nblk = 0, nbuf = 2;
  int ra = 1;                // batches of tap reads issued ahead of the FMAs
  int cb = 0;                // 1: a read batch is a channel's steps (ds_read2_b32 pairs from a
                             // per-channel base register); 0: one step (ds_read_b32)
  int seq = 0;               // 1: each workgroup runs every group in turn (the stores of one
                             // group overlap the next group's copies and FMAs); 0: one group
                             // per workgroup
  int gw = 0;                // 1: the workgroup holds every group's wavefronts (T tiles x G
                             // groups), which share the staged window
  int pairdist = 0;          // 1: of the W = wpb() wavefronts that share a window, wave w
                             // stages block w % nblk of every (W / nblk)-th channel
  int c0 = 0;                // channels of the first chunk (0: Cc); later chunks double up to Cc
  int es = 0;                // early stores: an output channel whose last FMA is in unit u is
                             // stored at the start of unit u + 1 (-1), or not before the group's
                             // es-th unit from the end (es >= 0; 0: after the last unit)
  int esnt = 0;              // cache policy of the early stores: 0 default, 1 nt, 2 sc0 sc1, 3 sc1
  int pb = 0;                // channel batches: one LDS base register per chunk slot and buffer,
                             // set once (else a base is made per channel)
  int vt = 0;                // VGPR target of the unstaged plans' groups and load depth (0: 168,
                             // three wavefronts per SIMD)
  long long fmas = 0;        // FMA instructions over all sections (= nnz)
  long long code_bytes = 0;  // size of the generated instruction stream
  long long sec_valu = 0;    // VALU instructions of the longest section (FMAs, shifts, reduction)
  long long sec_steps = 0;   // load steps of the longest section
  long long sec_loads = 0;   // row loads of the section with the most
  std::vector<std::vector<int>> rows;  // output channels of each group
  int wpb() const { return stage && gw ? T * G : Q * T; }
};

// Kernel arguments, in the order of the kernel's argument segment (40 bytes).
struct BakeArgs {
  uint64_t x, y;      // input and output base addresses
  uint32_t N;         // images
  uint32_t ntiles;    // wavefront tiles: ceil(N*E*Pb / V)
  uint32_t x_bytes;   // N*C*H*W*4: range of the input descriptor (< 2^31)
  uint32_t y_bytes;   // N*M*E*F*4: range of the output descriptor (< 2^31)
  uint32_t qtot;      // N*E*Pb
  uint32_t per_xcd;   // workgroups per XCD (the grid is 8*per_xcd workgroups)
};

// Options from SPARSECONV_BAKE="G=..,Q=..,T=..,D=..,DPP=..,PERM=..,STAGE=..,NB=..,CC=..,RA=..,CB=..,SEQ=..,GW=..,C0=..,ES=..,ESNT=..,ORD=..,VT=..,PB=.." (tuning and
// tests only); fields left at -1 are chosen by the packer.
struct BakeForce {
  int G = -1, Q = -1, T = -1, D = -1, dpp = -1, perm = -1, stage = -1, nb = -1, cc = -1, ra = -1, cb = -1,
      seq = -1, gw = -1, c0 = -1, es = -2, esnt = -1, vt = -1, pb = -1;
  bool any() const {
    return G > 0 || Q > 0 || T > 0 || D > 0 || dpp >= 0 || perm >= 0 || stage >= 0 || nb > 0 || cc > 0 || ra > 0 ||
           cb >= 0 || seq >= 0 || gw >= 0 || c0 >= 0 || es >= -1 || esnt >= 0 || vt > 0 || pb >= 0;
  }
};
BakeForce bake_force_from_env();

// The plans a handle generates kernels for: one when forced, else the base plan (the fewest
// groups that fit registers and instruction cache) and variants with more wavefronts per
// unit of work (channel splits, more groups, one unit per workgroup) for small batches.
// Empty (with *why) if the layer does not fit the mapping.
std::vector<BakePlan> bake_candidates(const Geom& g, const std::vector<int32_t>& rowptr,
                                      const std::vector<int32_t>& col, const BakeForce& f, std::string* why);

// Estimated cycles of a forward of N images with plan p on `cus` compute units (ranks the
// handle's kernels; the constants are fitted to MI355X measurements).
double bake_estimate(const Geom& g, const BakePlan& p, int N, int cus);

// Generate the GCN assembly of a plan's kernel (symbol "sc_baked").
bool bake_generate(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                   const std::vector<float>& val, BakePlan* plan, std::string* src, std::string* err);

// Assemble and link with amd_comgr into a code object for gfx950.
bool bake_assemble(const std::string& src, std::vector<char>* elf, std::string* err);

// Magic numbers for q = mulhi(n, m) >> l == n / d for every n < 2^31 (d >= 2).
void bake_magic(uint32_t d, uint32_t* m, int* l);

}  // namespace sc
