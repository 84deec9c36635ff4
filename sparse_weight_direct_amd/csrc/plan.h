// Internal types shared by the packer, the C ABI and the gfx950 kernels.
//
// Data layout used by the kernels (all sizes in 4-byte words):
//
//  * The padded input of one image is split into stride x stride phase planes: padded
//    position (yp, xp) lands in phase (yp % st, xp % st) at phase coordinates
//    (yp / st, xp / st).  A phase plane has HYp = ceil((H+2p)/st) rows of Pp = ceil((W+2p)/st)
//    words.  For stride 1 this is just the zero-padded image.
//  * Output (e, f) of image n reads, for tap (r, s), phase (r % st, s % st) at
//    (e + r/st, f + s/st): with stride folded into the phases every tap is a unit-stride
//    shift, so a run of consecutive "extended" output indices I = n*HYp*Pp + e*Pp + f maps
//    to consecutive LDS words for every tap.  Positions with e >= E or f >= F are junk
//    (computed, never stored).
//  * A workgroup owns 64*K consecutive extended indices (K per lane, 64 apart) and stages
//    the phase rows they touch, NRmax rows per phase, for Cc channels at a time:
//        LDS word = c_l*CHS + (py*st + px)*PH + row*Pp + col,  PH = NRmax*Pp,
//    with the channel stride CHS = st*st*PH rounded up to a multiple of 64 words, so that
//    every channel is nblk = CHS/64 blocks of 64 words and a block's source offsets are
//    the same for every channel (they differ by a multiple of H*W).
//  * Each stored non-zero (c, r, s, v) is re-encoded at pack time as
//        enc = (c % Cc)*CHS + ((r % st)*st + (s % st))*PH + (r / st)*Pp + (s / st)
//    so the inner loop is: one address add, K LDS reads 64 words apart, K FMAs.
#pragma once
#include <cstdint>
#include <vector>

namespace sc {

constexpr int kLdsMax = 160 * 1024;     // LDS per CU

struct Geom {
  int M, C, R, S, H, W, st, pad;
  int E, F;        // output extent
  int Pp, HYp;     // phase plane row pitch and rows per image
  int Rr;          // distinct r / st values = (R-1)/st + 1
};

struct Plan {
  int K;           // extended output positions per lane (64 apart)
  int OCW;         // output-channel slots per wavefront
  int NW;          // wavefronts per workgroup (8 or 16)
  int G;           // output-channel groups (work units per tile)
  int Cc;          // channels staged per chunk
  int nch;         // number of chunks = ceil(C / Cc)
  int NRmax;       // phase rows staged per phase plane
  int PH;          // words per phase plane = NRmax * Pp
  int CHS;         // words per staged channel = st*st*PH rounded up to a multiple of 64
  int nblk;        // 64-word blocks per staged channel = CHS / 64
  int rt;          // row-table entries per wavefront (>= st*NRmax, multiple of 64)
  int QE;          // loads of 64 words per wavefront per step carrying its block of
                   // non-zeros (32 entries each)
  int nin;         // words of a ring slot holding input rows (Cc*CHS + read slack)
  int slot_words;  // words of one ring slot = nin + QE*64*NW
  int lds_bytes;   // two ring slots + per-wavefront row tables + block-start table
  int span_images; // most images one tile's staged rows can touch
};

// Kernel arguments (by value).
struct KArgs {
  const float* x;
  float* y;
  const uint32_t* ent;    // sparse: pairs {enc, value bits}
  const int32_t* seg;     // sparse: [(group*NW + wave)*(nch+1) + k] -> first entry of block k
  const int* slot_row;    // sparse: [group][wave][slot] -> output channel or -1
  int N, C, H, W, M, E, F, R, S, st, pad;
  int Pp, HYp, img_ext;   // img_ext = HYp * Pp
  int NRmax, PH, CHS, nblk, Cc, nch, G, rt, QE, nin, slot_words;
  int HW;                 // H * W
  int ntiles;             // tiles of 64*K extended positions
  long long x_words;      // N * C * H * W
  long long ext_total;    // N * img_ext
};

bool make_geom(int M, int C, int R, int S, int H, int W, int st, int pad, Geom* g);
// Launch plan for the CSR filter matrix (rowptr, col): also schedules rows onto wavefront
// slots (slot_row) and sizes each wavefront's per-chunk block of non-zeros.
Plan choose_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 std::vector<int32_t>* slot_row, int32_t* max_wave_nnz);
int plan_nrmax(const Geom& g, int K);

// Header entries at the start of a wavefront's per-chunk block of non-zeros.
int block_header(int OCW);

// Workgroups to launch for `units` work units: every CU busy, each workgroup a contiguous
// run of units (kernels.hip; uses the occupancy of the chosen kernel).
int grid_size(const Plan& p, long long units, int* err);

// Launchers (kernels.hip).  Return a hipError_t value as int.
int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks);

}  // namespace sc
